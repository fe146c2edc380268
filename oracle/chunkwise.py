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

``backward`` is the gradient of the same function in the chunk-level form the
GPU gradient kernel uses (no pass inside a chunk is serial): given every
chunk's entry state S (forward over the chunks) and exit gradient dS' (the
adjoint recurrence dS = diag(e^Ge) dS' + Qs^T dO - W^T dU, last chunk first),
  dO = dY sigmoid(z),  dU = Kp dS' + P^T dO,  dQs = dO S^T,  dW = -dU S^T,
  dKp = U dS'^T,  dP = lower_incl(dO U^T),  dX = T^T dW,  dY~ = T^T dU,
  dA = strict_lower(-dX W^T - dY~ U~^T)   (= -T^T dT T^T with dT = dW X^T + dU Y^T),
with Qs = scale Q e^G, Ks = K e^G, Kp = K e^{Ge - G}, X = diag(beta) Ks,
Y = diag(beta) V.  The products with the blocks of M = A / beta and P are
taken over 16-token blocks with references B_I = G before block I: block
(I, J) uses the row factors K_I e^{G - B_I}, scale Q_I e^{G - B_I} and the
column factors K_J e^{B_I - G}, and the column gradients use the row factors
K_I e^{G - B_J}; every factor stays in range when g >= -5 (the chunk path's
floor).  dg is the suffix sum of the per-token dG plus dGe.
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


def _chunk_bwd(q, k, v, g, beta, z, dy, S, dSn, scale, sub):
    """Gradients of one chunk (rows past its end zero-padded by the caller) and
    dS on its entry; the chunk length is a multiple of ``sub``."""
    C = k.shape[0]
    nb = C // sub
    G = np.cumsum(g, axis=0)
    Ge = G[C - 1]
    B = np.zeros((nb, k.shape[1]))
    for i in range(1, nb):
        B[i] = G[sub * i - 1]
    blk = lambda i: slice(sub * i, sub * i + sub)
    # forward quantities, blocks of M and P with the row block's reference
    M = np.zeros((C, C))
    P = np.zeros((C, C))
    for i in range(nb):
        kr = k[blk(i)] * np.exp(G[blk(i)] - B[i])
        qr = scale * q[blk(i)] * np.exp(G[blk(i)] - B[i])
        for j in range(i + 1):
            kc = k[blk(j)] * np.exp(B[i] - G[blk(j)])
            M[blk(i), blk(j)] = kr @ kc.T
            P[blk(i), blk(j)] = qr @ kc.T
    M = np.tril(M, -1)
    P = np.tril(P)
    T = np.linalg.inv(np.eye(C) + beta[:, None] * M)
    Ks = k * np.exp(G)
    Kp = k * np.exp(Ge - G)
    Qs = scale * q * np.exp(G)
    W = T @ (beta[:, None] * Ks)
    Ut = T @ (beta[:, None] * v)
    U = Ut - W @ S
    O = Qs @ S + P @ U
    # backward
    sg = _sigmoid(z)
    dO = dy * sg
    dz = dy * O * sg * (1.0 - sg)
    dU = Kp @ dSn + P.T @ dO
    dQs = dO @ S.T
    dW = -dU @ S.T
    dKp = U @ dSn.T
    dP = np.tril(dO @ U.T)
    dX = T.T @ dW
    dYt = T.T @ dU
    dA = np.tril(-dX @ W.T - dYt @ Ut.T, -1)
    dS = np.exp(Ge)[:, None] * dSn + Qs.T @ dO - W.T @ dU
    dq = scale * np.exp(G) * dQs
    dk = np.exp(G) * beta[:, None] * dX + np.exp(Ge - G) * dKp
    dv = beta[:, None] * dYt
    dG = Qs * dQs + Ks * beta[:, None] * dX - Kp * dKp
    dbeta = (dX * Ks).sum(1) + (dYt * v).sum(1)
    for i in range(nb):                               # row gradients of block row i
        egb = np.exp(G[blk(i)] - B[i])
        kr, qr = k[blk(i)] * egb, scale * q[blk(i)] * egb
        Z = sum(dA[blk(i), blk(j)] @ (k[blk(j)] * np.exp(B[i] - G[blk(j)])) for j in range(i + 1))
        dQr = sum(dP[blk(i), blk(j)] @ (k[blk(j)] * np.exp(B[i] - G[blk(j)])) for j in range(i + 1))
        dKr = beta[blk(i), None] * Z
        dbeta[blk(i)] += (kr * Z).sum(1)             # the dA . M term of dbeta
        dq[blk(i)] += scale * egb * dQr
        dk[blk(i)] += egb * dKr
        dG[blk(i)] += qr * dQr + kr * dKr
    for j in range(nb):                               # column gradients of block column j
        ebg = np.exp(B[j] - G[blk(j)])
        dKc = sum((beta[blk(i), None] * dA[blk(i), blk(j)]).T @ (k[blk(i)] * np.exp(G[blk(i)] - B[j]))
                  + dP[blk(i), blk(j)].T @ (scale * q[blk(i)] * np.exp(G[blk(i)] - B[j]))
                  for i in range(j, nb))
        dk[blk(j)] += ebg * dKc
        dG[blk(j)] -= k[blk(j)] * ebg * dKc
    dGe = (Kp * dKp).sum(0) + np.exp(Ge) * (dSn * S).sum(1)
    dg = np.cumsum(dG[::-1], axis=0)[::-1] + dGe
    S_next = np.exp(Ge)[:, None] * S + Kp.T @ U
    return dict(dq=dq, dk=dk, dv=dv, dg=dg, dbeta=dbeta, dz=dz), dS, S_next


def backward(q, k, v, g, beta, z, dout, init_state=None, dfinal=None, cu_seqlens=None,
             chunk=64, sub=16, scale=1.0):
    """Same interface and result as ``oracle.backward`` (packed [T, H, d] only),
    in the chunk-level form above; ``chunk`` is a multiple of ``sub``."""
    q, k, v, g, z, dout = (np.asarray(x, dtype=np.float64) for x in (q, k, v, g, z, dout))
    beta = np.asarray(beta, dtype=np.float64)
    T, H, dk = q.shape
    dv = v.shape[2]
    cu = np.array([0, T]) if cu_seqlens is None else np.asarray(cu_seqlens, dtype=np.int64)
    N = len(cu) - 1
    res = {n: np.zeros(q.shape) for n in ("dq", "dk", "dg")}
    res["dv"] = np.zeros(v.shape)
    res["dz"] = np.zeros(v.shape)
    res["dbeta"] = np.zeros((T, H))
    res["dinit"] = np.zeros((N, H, dk, dv))
    for n in range(N):
        a, e = int(cu[n]), int(cu[n + 1])
        nch = (e - a + chunk - 1) // chunk
        for h in range(H):
            def pad(x, j):
                lo, hi = a + j * chunk, min(a + j * chunk + chunk, e)
                y = np.zeros((chunk,) + x.shape[2:])
                y[:hi - lo] = x[lo:hi, h]
                return y
            S = np.zeros((dk, dv)) if init_state is None else np.array(init_state[n, h], dtype=np.float64)
            states = []
            for j in range(nch):                      # entry state of every chunk
                states.append(S)
                *_, S = _chunk_bwd(pad(q, j), pad(k, j), pad(v, j), pad(g, j), pad(beta, j),
                                   pad(z, j), np.zeros((chunk, dv)), S, np.zeros((dk, dv)), scale, sub)
            dSn = np.zeros((dk, dv)) if dfinal is None else np.array(dfinal[n, h], dtype=np.float64)
            for j in reversed(range(nch)):            # exit gradients, last chunk first
                gr, dSn, _ = _chunk_bwd(pad(q, j), pad(k, j), pad(v, j), pad(g, j), pad(beta, j),
                                        pad(z, j), pad(dout, j), states[j], dSn, scale, sub)
                lo, hi = a + j * chunk, min(a + j * chunk + chunk, e)
                for key in ("dq", "dk", "dg", "dv", "dz", "dbeta"):
                    res[key][lo:hi, h] = gr[key][:hi - lo]
            res["dinit"][n, h] = dSn
    return res
