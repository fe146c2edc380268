"""Pins for the oracle's backward (reverse-mode gradients of the recurrence).

* central finite differences of the loss sum(dout * out) + sum(dfinal * final)
  in fp64, for every input element, on small cases that cross the 32-token
  recompute segments, with varlen packing, an initial state and scale != 1;
* Euler's identity: out and the final state are jointly linear in (v, S0), so
  <dL/dv, v> + <dL/dS0, S0> = L exactly;
* the gate's closed form: dz = dout * out * (1 - sigmoid(z));
* the chunk-level form (``oracle.chunkwise.backward``: entry states and exit
  gradients per chunk, blockwise token products with block-start references)
  equals the token-by-token backward, on ragged varlen packing with empty,
  one-token and exactly-one-chunk sequences, a channel pinned at the gate
  floor and a no-decay stretch.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from oracle import chunkwise


def case(seed, lengths, H, dk, dv, init=True):
    rng = np.random.default_rng(seed)
    T = sum(lengths)
    x = {"q": rng.standard_normal((T, H, dk)), "k": rng.standard_normal((T, H, dk)) * 0.7,
         "v": rng.standard_normal((T, H, dv)), "g": -rng.random((T, H, dk)) * 1.5,
         "beta": rng.random((T, H)), "z": rng.standard_normal((T, H, dv))}
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    N = len(lengths)
    s0 = rng.standard_normal((N, H, dk, dv)) * 0.5 if init else None
    dy = rng.standard_normal((T, H, dv))
    df = rng.standard_normal((N, H, dk, dv))
    return x, cu, s0, dy, df


def loss(x, cu, s0, dy, df, scale):
    out, fin = oracle.forward(x["q"], x["k"], x["v"], x["g"], x["beta"], x["z"],
                              init_state=s0, cu_seqlens=cu, scale=scale)
    return float(np.sum(out * dy) + np.sum(fin * df))


@pytest.mark.parametrize("seed,lengths,H,dk,dv,scale", [
    (0, [5], 2, 3, 2, 1.0),
    (1, [3, 0, 4], 1, 2, 3, 0.7),
    (2, [37], 1, 2, 2, 1.3),          # crosses a 32-token recompute segment
])
def test_backward_matches_finite_differences(seed, lengths, H, dk, dv, scale):
    x, cu, s0, dy, df = case(seed, lengths, H, dk, dv)
    r = oracle.backward(x["q"], x["k"], x["v"], x["g"], x["beta"], x["z"], dy, init_state=s0,
                        dfinal=df, cu_seqlens=cu, scale=scale)
    h = 1e-6
    pairs = [(name, "d" + name) for name in ("q", "k", "v", "g", "beta", "z")] + [("s0", "dinit")]
    for name, key in pairs:
        base = s0 if name == "s0" else x[name]
        fd = np.zeros_like(base)
        for idx in np.ndindex(base.shape):
            hi, lo = base.copy(), base.copy()
            hi[idx] += h
            lo[idx] -= h
            if name == "s0":
                lp, lm = loss(x, cu, hi, dy, df, scale), loss(x, cu, lo, dy, df, scale)
            else:
                lp = loss(dict(x, **{name: hi}), cu, s0, dy, df, scale)
                lm = loss(dict(x, **{name: lo}), cu, s0, dy, df, scale)
            fd[idx] = (lp - lm) / (2 * h)
        err = np.max(np.abs(fd - r[key])) / max(np.max(np.abs(fd)), 1e-12)
        assert err < 1e-6, f"{key}: finite-difference mismatch {err}"


def test_euler_identity_in_values_and_initial_state():
    x, cu, s0, dy, df = case(5, [40, 9], 2, 4, 3)
    r = oracle.backward(x["q"], x["k"], x["v"], x["g"], x["beta"], x["z"], dy, init_state=s0,
                        dfinal=df, cu_seqlens=cu)
    lhs = float(np.sum(r["dv"] * x["v"]) + np.sum(r["dinit"] * s0))
    rhs = loss(x, cu, s0, dy, df, 1.0)
    assert abs(lhs - rhs) <= 1e-10 * max(1.0, abs(rhs))


def test_gate_gradient_closed_form():
    x, cu, s0, dy, df = case(6, [20], 2, 3, 3)
    out, _ = oracle.forward(x["q"], x["k"], x["v"], x["g"], x["beta"], x["z"], init_state=s0,
                            cu_seqlens=cu)
    r = oracle.backward(x["q"], x["k"], x["v"], x["g"], x["beta"], x["z"], dy, init_state=s0,
                        cu_seqlens=cu)
    sg = 1.0 / (1.0 + np.exp(-x["z"]))
    np.testing.assert_allclose(r["dz"], dy * out * (1.0 - sg), rtol=1e-12, atol=1e-14)


def test_no_final_gradient_and_zero_init_are_defaults():
    x, cu, _, dy, _ = case(7, [6], 1, 2, 2, init=False)
    r = oracle.backward(x["q"], x["k"], x["v"], x["g"], x["beta"], x["z"], dy, cu_seqlens=cu)
    r0 = oracle.backward(x["q"], x["k"], x["v"], x["g"], x["beta"], x["z"], dy, cu_seqlens=cu,
                         init_state=np.zeros((1, 1, 2, 2)), dfinal=np.zeros((1, 1, 2, 2)))
    for key in r:
        np.testing.assert_array_equal(r[key], r0[key])


@pytest.mark.parametrize("chunk,sub", [(64, 16), (32, 8), (16, 16), (16, 4)])
def test_chunk_level_form_equals_token_backward(chunk, sub):
    lengths = [150, 0, 64, 1, 17, 65]
    x, cu, s0, dy, df = case(20 + chunk, lengths, 2, 8, 6)
    rng = np.random.default_rng(chunk)
    x["g"] = rng.uniform(-5.0, 0.0, x["g"].shape)
    x["g"][20:110, 1, 3] = -5.0                   # a channel pinned at the floor
    x["g"][160:190, 0, :] = 0.0                   # no decay
    args = (x["q"], x["k"], x["v"], x["g"], x["beta"], x["z"], dy)
    ref = oracle.backward(*args, init_state=s0, dfinal=df, cu_seqlens=cu, scale=0.8)
    got = chunkwise.backward(*args, init_state=s0, dfinal=df, cu_seqlens=cu, chunk=chunk,
                             sub=sub, scale=0.8)
    for key in ("dq", "dk", "dv", "dg", "dbeta", "dz", "dinit"):
        err = np.max(np.abs(got[key] - ref[key])) / max(np.max(np.abs(ref[key])), 1e-30)
        assert err < 1e-10, f"{key}: {err}"
