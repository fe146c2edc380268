"""Exact rational brute force for KDA on tiny inputs -- test infrastructure only.

Written in the dense matrix form of one KDA token, which is an algebraic
rewrite of predict-subtract-write (so a slip in either form shows up as a
mismatch):
    S_t = (I - beta_t k_t k_t^T) diag(a_t) S_{t-1} + beta_t k_t v_t^T
    y_t = gate_t * (scale S_t^T q_t)
with a_t = exp(g_t) supplied directly as rationals (a = 0 stands for
g = -inf) and gate_t = sigmoid(z_t) supplied as rationals in (0, 1).
Source: "Kimi K3 second-pass study ledger", section 1, rows Q04 and Q05
(delta-rule write with channel-wise decay), row Q08 (output gate).
All arithmetic is in ``fractions.Fraction``; there is no rounding at all.
"""
from __future__ import annotations

from fractions import Fraction


def _matmul(A, B):
    n, m, p = len(A), len(B), len(B[0])
    return [[sum((A[i][t] * B[t][j] for t in range(m)), Fraction(0)) for j in range(p)]
            for i in range(n)]


def token(S, q, k, v, a, beta, gate, scale=Fraction(1)):
    """One token on state S (list of dk rows of dv Fractions). Returns (S', y)."""
    dk, dv = len(S), len(S[0])
    # H = I - beta k k^T ;  D = diag(a)
    Hm = [[(Fraction(1) if i == j else Fraction(0)) - beta * k[i] * k[j] for j in range(dk)]
          for i in range(dk)]
    DS = [[a[i] * S[i][j] for j in range(dv)] for i in range(dk)]
    Sn = _matmul(Hm, DS)
    Sn = [[Sn[i][j] + beta * k[i] * v[j] for j in range(dv)] for i in range(dk)]
    y = [gate[j] * scale * sum((Sn[i][j] * q[i] for i in range(dk)), Fraction(0))
         for j in range(dv)]
    return Sn, y


def forward(seqs, S0=None, scale=Fraction(1)):
    """``seqs``: list of tokens, each a dict with q, k, a (len dk), v, gate
    (len dv) and beta, all Fractions.  Returns (list of y, final S)."""
    dk = len(seqs[0]["k"]) if seqs else len(S0)
    dv = len(seqs[0]["v"]) if seqs else len(S0[0])
    S = [[Fraction(0)] * dv for _ in range(dk)] if S0 is None else [list(r) for r in S0]
    ys = []
    for tok in seqs:
        S, y = token(S, tok["q"], tok["k"], tok["v"], tok["a"], tok["beta"], tok["gate"], scale)
        ys.append(y)
    return ys, S
