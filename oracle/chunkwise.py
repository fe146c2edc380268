"""Chunkwise-parallel form of KDA in fp64 NumPy -- test infrastructure only.

A second, independent implementation of the same function as the recurrent
oracle, written the way the pages describe the fast form: the sequence is cut
into chunks, the state is passed recurrently from one chunk to the next, and
inside a chunk everything is dense matrix work ("Kimi K3 second-pass study
ledger", section 1, row Q07; "Kimi K3 report reveals training and systems
stack", confirmed list, FlashKDA item).

Derivation (per chunk of L tokens with entry state S; r, s index tokens inside
the chunk, decays are per key channel):
  G_r          = sum of g over chunk tokens 1..r (inclusive)
  D[r, s]      = sum of g over tokens s+1..r (s < r); the decay from s to r
  A[r, s]      = sum_c k_r[c] k_s[c] exp(D[r, s, c])         for s < r
  P[r, s]      = sum_c q_r[c] k_s[c] exp(D[r, s, c])         for s <= r
  T            = (I + diag(beta) A)^-1
  W            = T diag(beta) (K * exp(G))        Ut = T diag(beta) V
  U            = Ut - W S                          (corrected values)
  O            = scale * ((Q * exp(G)) S + P U),   y = sigmoid(z) * O
  S_next       = diag(exp(G_L)) S + (K * exp(G_L - G))^T U
Decay ratios are built from interval sums of g (never exp(G_r) * exp(-G_s)),
so g = -inf gives exact zeros instead of inf * 0.
"""
from __future__ import annotations

import numpy as np


def _sigmoid(x):
    return 1.0 / (1.0 + np.exp(-x))


def _chunk(q, k, v, g, beta, z, S, scale):
    """One chunk: q, k, g [L, dk]; v, z [L, dv]; beta [L]; S [dk, dv]."""
    L, dk = k.shape
    G = np.cumsum(g, axis=0)                      # inclusive, from chunk start
    D = np.full((L, L, dk), -np.inf)              # D[r, s] for s <= r
    for s in range(L):
        D[s, s] = 0.0
        if s + 1 < L:
            D[s + 1:, s] = np.cumsum(g[s + 1:], axis=0)
    E = np.exp(D)                                 # decay from s to r; 0 above the diagonal
    A = np.einsum("rc,sc,rsc->rs", k, k, E)
    A = np.tril(A, -1)
    P = np.einsum("rc,sc,rsc->rs", q, k, E)
    P = np.tril(P)
    T = np.linalg.inv(np.eye(L) + beta[:, None] * A)
    W = T @ (beta[:, None] * (k * np.exp(G)))
    Ut = T @ (beta[:, None] * v)
    U = Ut - W @ S
    O = scale * ((q * np.exp(G)) @ S + P @ U)
    y = _sigmoid(z) * O
    tail = E[L - 1]                               # decay from each s to the chunk end
    S_next = np.exp(G[L - 1])[:, None] * S + (k * tail).T @ U
    return y, S_next


def forward(q, k, v, g, beta, z, init_state=None, cu_seqlens=None, chunk=16, scale=1.0):
    """Same interface and result as ``oracle.forward`` (packed [T, H, d] or
    batched [B, T, H, d]); ``chunk`` is the chunk length (any positive int;
    the last chunk of a sequence may be partial)."""
    q = np.asarray(q, dtype=np.float64)
    batched = q.ndim == 4
    if batched:
        B, T, H, dk = q.shape
    else:
        B = 1
        T, H, dk = q.shape
    dv = np.asarray(v).shape[-1]
    r = lambda x, d: np.asarray(x, dtype=np.float64).reshape((B * T, H, d) if d else (B * T, H))
    q, k, g = r(q, dk), r(k, dk), r(g, dk)
    v, z = r(v, dv), r(z, dv)
    beta = r(beta, 0)
    cu = (np.arange(B + 1) * T) if cu_seqlens is None else np.asarray(cu_seqlens, dtype=np.int64)
    N = len(cu) - 1
    out = np.zeros((B * T, H, dv))
    final = np.zeros((N, H, dk, dv))
    for n in range(N):
        for h in range(H):
            S = np.zeros((dk, dv)) if init_state is None else np.array(init_state[n, h], dtype=np.float64)
            for c0 in range(int(cu[n]), int(cu[n + 1]), chunk):
                c1 = min(c0 + chunk, int(cu[n + 1]))
                sl = slice(c0, c1)
                y, S = _chunk(q[sl, h], k[sl, h], v[sl, h], g[sl, h], beta[sl, h], z[sl, h], S, scale)
                out[sl, h] = y
            final[n, h] = S
    out = out.reshape(B, T, H, dv) if batched else out.reshape(T, H, dv)
    return out, final
