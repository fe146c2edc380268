"""Oracle of the optional input prologue -- test infrastructure only.

The fused prologue lets callers hand the kernels raw projections instead of
the prepared inputs of the recurrence:

  * q, k: L2-normalised over the key dimension per (token, head), with a small
    epsilon inside the square root: x / sqrt(sum(x^2) + 1e-6);
  * beta: a logit, mapped to sigmoid(beta) in (0, 1);
  * g: a pre-activation x, mapped to the log-decay max(-5, -softplus(x)),
    softplus(x) = log(1 + exp(x)), so that the decay is at most 1 and the
    log-decay never goes below the floor -5.

Source: "Kimi K3 second-pass study ledger" (llm-atlas K3_RESEARCH.md),
section 1 row Q06 (log-decay floor g_min = -5).  The pages do not say how q,
k, beta and g are produced from the layer's projections; normalised keys, a
sigmoid write strength and a softplus-based log-decay are the readings taken
here (the same maps the synthetic workloads use to draw their inputs).
Parity is pinned against closed forms and identities in
``tests/test_oracle_prologue.py``.

All functions work in float64 on NumPy arrays; nothing here is shared with
the HIP path.
"""
from __future__ import annotations

import numpy as np

G_MIN = -5.0
NORM_EPS = 1e-6

QK_L2NORM = 1
BETA_SIGMOID = 2
G_SOFTPLUS = 4


def l2norm(x):
    """x / sqrt(sum(x^2, last axis) + NORM_EPS), in float64."""
    x = np.asarray(x, dtype=np.float64)
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + NORM_EPS)


def sigmoid(x):
    """1 / (1 + exp(-x)), evaluated without overflow for large |x|."""
    x = np.asarray(x, dtype=np.float64)
    e = np.exp(-np.abs(x))
    return np.where(x >= 0, 1.0 / (1.0 + e), e / (1.0 + e))


def softplus(x):
    """log(1 + exp(x)) = max(x, 0) + log1p(exp(-|x|))."""
    x = np.asarray(x, dtype=np.float64)
    return np.maximum(x, 0.0) + np.log1p(np.exp(-np.abs(x)))


def log_decay(x):
    """max(G_MIN, -softplus(x))."""
    return np.maximum(G_MIN, -softplus(x))


def apply(q, k, beta, g, flags):
    """The prepared (q, k, beta, g) in float64 for the given prologue flags
    (a combination of QK_L2NORM, BETA_SIGMOID and G_SOFTPLUS)."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    beta = np.asarray(beta, dtype=np.float64)
    g = np.asarray(g, dtype=np.float64)
    if flags & QK_L2NORM:
        q, k = l2norm(q), l2norm(k)
    if flags & BETA_SIGMOID:
        beta = sigmoid(beta)
    if flags & G_SOFTPLUS:
        g = log_decay(g)
    return q, k, beta, g
