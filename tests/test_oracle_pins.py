"""Pins for the CPU oracle: each check ties it to something other than itself.

* exact rational brute force in the dense matrix form (``oracle.exact``);
* hand-worked examples under ``tests/golden`` (Lab A, decay order, Lab B);
* closed forms: beta = 0 (pure decay and read), dk = 1 (a gated EMA);
* invariants: orthonormal-key retrieval, reset by g = -inf, chunkwise form ==
  recurrence, split/concat of sequences, decode steps == forward, linearity
  in (S0, V), dv-column separability, a norm bound.

Sources: "Kimi K3 second-pass study ledger" (llm-atlas K3_RESEARCH.md),
section 1 rows Q04-Q08 and section 5 Labs A and B; "Kimi K3 report reveals
training and systems stack" (FlashKDA, 16-token tiles).
"""
from __future__ import annotations

import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle import chunkwise, exact

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ----------------------------------------------------------------- helpers
def rel_err(x, ref):
    x, ref = np.asarray(x, dtype=np.float64), np.asarray(ref, dtype=np.float64)
    den = np.max(np.abs(ref))
    return float(np.max(np.abs(x - ref)) / (den if den > 0 else 1.0))


def random_inputs(rng, T, H, dk, dv, g_lo=-5.0, unit_keys=True):
    q = rng.standard_normal((T, H, dk))
    k = rng.standard_normal((T, H, dk))
    if unit_keys:
        q /= np.linalg.norm(q, axis=-1, keepdims=True)
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((T, H, dv))
    g = rng.uniform(g_lo, 0.0, (T, H, dk))
    beta = rng.uniform(0.0, 1.0, (T, H))
    z = rng.standard_normal((T, H, dv))
    return q, k, v, g, beta, z


def logit(p):
    return math.log(p / (1.0 - p))


def rational_case(seed, lens, H, dk, dv):
    """Random tiny rational inputs.  Returns (float arrays for the oracle,
    per-(seq, head) token dicts for the exact form, S0 rationals)."""
    rng = np.random.default_rng(seed)
    T = sum(lens)
    fr = lambda: Fraction(int(rng.integers(-8, 9)), int(rng.choice([1, 2, 4, 8])))
    a_choices = [Fraction(0), Fraction(1, 4), Fraction(1, 2), Fraction(3, 4), Fraction(1)]
    b_choices = [Fraction(0), Fraction(1, 4), Fraction(1, 2), Fraction(1)]
    gate_choices = [Fraction(1, 4), Fraction(1, 2), Fraction(3, 4)]
    toks = [[dict(q=[fr() for _ in range(dk)], k=[fr() for _ in range(dk)],
                  v=[fr() for _ in range(dv)],
                  a=[a_choices[int(rng.integers(0, 5))] for _ in range(dk)],
                  beta=b_choices[int(rng.integers(0, 4))],
                  gate=[gate_choices[int(rng.integers(0, 3))] for _ in range(dv)])
             for _ in range(H)] for _ in range(T)]
    S0 = [[[[fr() for _ in range(dv)] for _ in range(dk)] for _ in range(H)] for _ in lens]
    f = lambda x: float(x)
    q = np.array([[[f(x) for x in toks[t][h]["q"]] for h in range(H)] for t in range(T)])
    k = np.array([[[f(x) for x in toks[t][h]["k"]] for h in range(H)] for t in range(T)])
    v = np.array([[[f(x) for x in toks[t][h]["v"]] for h in range(H)] for t in range(T)])
    g = np.array([[[(-np.inf if x == 0 else math.log(x)) for x in toks[t][h]["a"]]
                   for h in range(H)] for t in range(T)])
    beta = np.array([[f(toks[t][h]["beta"]) for h in range(H)] for t in range(T)])
    z = np.array([[[logit(f(x)) for x in toks[t][h]["gate"]] for h in range(H)]
                  for t in range(T)])
    init = np.array([[[[f(x) for x in row] for row in S0[n][h]] for h in range(H)]
                     for n in range(len(lens))])
    return (q, k, v, g, beta, z, init), toks, S0


# ----------------------------------------------------- exact brute force
@pytest.mark.parametrize("seed,lens,H,dk,dv", [
    (0, [4], 1, 2, 2), (1, [3, 0, 2], 2, 3, 2), (2, [1, 4], 2, 1, 3), (3, [2, 2, 1], 1, 3, 3),
    (4, [5], 2, 2, 1),
])
def test_forward_matches_exact_rational(seed, lens, H, dk, dv):
    (q, k, v, g, beta, z, init), toks, S0 = rational_case(seed, lens, H, dk, dv)
    cu = np.concatenate([[0], np.cumsum(lens)])
    out, final = oracle.forward(q, k, v, g, beta, z, init_state=init, cu_seqlens=cu)
    for n in range(len(lens)):
        for h in range(H):
            seq = [toks[t][h] for t in range(cu[n], cu[n + 1])]
            ys, S = exact.forward(seq, S0=S0[n][h])
            for i, t in enumerate(range(cu[n], cu[n + 1])):
                np.testing.assert_allclose(out[t, h], [float(x) for x in ys[i]],
                                           rtol=1e-13, atol=1e-13)
            np.testing.assert_allclose(final[n, h], [[float(x) for x in r] for r in S],
                                       rtol=1e-13, atol=1e-13)


def test_decode_step_matches_exact_rational():
    (q, k, v, g, beta, z, init), toks, S0 = rational_case(11, [1, 1, 1], 2, 3, 2)
    state = np.ascontiguousarray(init)
    y = oracle.decode_step(q, k, v, g, beta, z, state)
    for n in range(3):
        for h in range(2):
            ys, S = exact.forward([toks[n][h]], S0=S0[n][h])
            np.testing.assert_allclose(y[n, h], [float(x) for x in ys[0]], rtol=1e-13, atol=1e-13)
            np.testing.assert_allclose(state[n, h], [[float(x) for x in r] for r in S],
                                       rtol=1e-13, atol=1e-13)


# ------------------------------------------------------------ golden files
def _read_golden(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as fh:
        for line in fh:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append([c.strip() for c in line.split("|")])
    return rows


def test_golden_lab_a_delta_vs_additive():
    for row in _read_golden("lab_a_repeated_key.txt"):
        beta = float(row[0].split()[1])
        y1 = [float(x) for x in row[1].split()]
        y2 = [float(x) for x in row[2].split()]
        fin = [[float(x) for x in r.split()] for r in row[3].split(";")]
        additive = [float(x) for x in row[4].split()]
        T, H, dk, dv = 2, 1, 2, 2
        q = np.array([[[1.0, 0.0]]] * T)
        k = np.array([[[1.0, 0.0]]] * T)
        v = np.array([[[1.0, 2.0]], [[3.0, -1.0]]])
        g = np.zeros((T, H, dk))
        b = np.full((T, H), beta)
        z = np.zeros((T, H, dv))
        out, final = oracle.forward(q, k, v, g, b, z)
        np.testing.assert_allclose(out[0, 0], y1, rtol=0, atol=1e-15)
        np.testing.assert_allclose(out[1, 0], y2, rtol=0, atol=1e-15)
        np.testing.assert_allclose(final[0, 0], fin, rtol=0, atol=1e-15)
        if beta == 1.0:
            # with beta = 1 the state returns the last value for the key, not the sum
            recall = final[0, 0].T @ np.array([1.0, 0.0])
            np.testing.assert_allclose(recall, v[1, 0], atol=1e-15)
            assert np.max(np.abs(recall - np.array(additive))) > 0.5


def test_golden_decay_order_two_tokens():
    d = {r[0]: [float(x) for x in r[1].split()] for r in _read_golden("decay_order_two_tokens.txt")}
    q = np.array([[d["q1"]], [d["q2"]]])
    k = np.array([[d["k1"]], [d["k2"]]])
    v = np.array([[[d["v"][0]]], [[d["v"][1]]]])
    g = np.log(np.array([[d["a1"]], [d["a2"]]]))
    beta = np.array([[d["beta"][0]], [d["beta"][1]]])
    z = np.array([[[logit(d["gate"][0])]], [[logit(d["gate"][1])]]])
    init = np.array(d["S0"]).reshape(1, 1, 2, 1)
    out, final = oracle.forward(q, k, v, g, beta, z, init_state=init)
    np.testing.assert_allclose(out[:, 0, 0], d["y"], rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(final[0, 0, :, 0], d["final"], rtol=1e-14, atol=1e-15)
    # the same case in exact arithmetic agrees with the hand values
    toks = [dict(q=[Fraction(x).limit_denominator(100) for x in d["q1"]],
                 k=[Fraction(x).limit_denominator(100) for x in d["k1"]],
                 v=[Fraction(3)], a=[Fraction(1, 2), Fraction(1, 4)], beta=Fraction(1),
                 gate=[Fraction(1, 2)]),
            dict(q=[Fraction(0), Fraction(1)], k=[Fraction(3, 5), Fraction(4, 5)],
                 v=[Fraction(1)], a=[Fraction(1), Fraction(1, 2)], beta=Fraction(1, 2),
                 gate=[Fraction(3, 4)])]
    ys, S = exact.forward(toks, S0=[[Fraction(2)], [Fraction(4)]])
    assert [y[0] for y in ys] == [Fraction(2), Fraction(3, 200)]
    assert [r[0] for r in S] == [Fraction(66, 25), Fraction(1, 50)]


def test_golden_lab_b_bound():
    import torch
    for row in _read_golden("lab_b_log_decay_bound.txt"):
        L = int(row[0])
        big = torch.tensor(5.0 * L, dtype=torch.float64).exp()
        small = torch.tensor(-5.0 * L, dtype=torch.float64).exp()
        bf_big = big.to(torch.bfloat16)
        fin_bf = bool(torch.isfinite(bf_big))
        normal_bf = bool(small >= torch.finfo(torch.bfloat16).tiny)
        fin_f16 = bool(big <= torch.finfo(torch.float16).max)
        assert fin_bf == (row[1] == "yes"), L
        assert normal_bf == (row[2] == "yes"), L
        assert fin_f16 == (row[3] == "yes"), L
    # 16 is the largest power-of-two tile whose worst reciprocal stays finite
    lmax = max(L for L in range(1, 64) if math.exp(5 * L) < float(torch.finfo(torch.bfloat16).max)
               and math.exp(-5 * L) >= float(torch.finfo(torch.bfloat16).tiny))
    assert lmax == 17 and 2 ** int(math.log2(lmax)) == 16


# ------------------------------------------------------------ closed forms
def test_beta_zero_is_pure_decay_and_read():
    rng = np.random.default_rng(5)
    T, H, dk, dv = 9, 2, 4, 3
    q, k, v, g, beta, z = random_inputs(rng, T, H, dk, dv)
    beta[:] = 0.0
    S0 = rng.standard_normal((1, H, dk, dv))
    out, final = oracle.forward(q, k, v, g, beta, z, init_state=S0, scale=0.7)
    Gam = np.cumsum(g, axis=0)                           # [T, H, dk]
    sig = 1.0 / (1.0 + np.exp(-z))
    for h in range(H):
        exp_out = sig[:, h] * 0.7 * ((q[:, h] * np.exp(Gam[:, h])) @ S0[0, h])
        np.testing.assert_allclose(out[:, h], exp_out, rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(final[0, h], np.exp(Gam[-1, h])[:, None] * S0[0, h],
                                   rtol=1e-12, atol=1e-14)


def test_dk1_is_gated_ema():
    rng = np.random.default_rng(6)
    T, H, dv = 12, 3, 5
    q = rng.standard_normal((T, H, 1))
    k = rng.standard_normal((T, H, 1))
    v = rng.standard_normal((T, H, dv))
    g = rng.uniform(-5, 0, (T, H, 1))
    beta = rng.uniform(0, 1, (T, H))
    z = rng.standard_normal((T, H, dv))
    S0 = rng.standard_normal((1, H, 1, dv))
    out, final = oracle.forward(q, k, v, g, beta, z, init_state=S0)
    for h in range(H):
        s = S0[0, h, 0].copy()
        for t in range(T):
            a, kk, b = math.exp(g[t, h, 0]), k[t, h, 0], beta[t, h]
            s = a * (1.0 - b * kk * kk) * s + b * kk * v[t, h]
            y = q[t, h, 0] * s / (1.0 + np.exp(-z[t, h]))
            np.testing.assert_allclose(out[t, h], y, rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(final[0, h, 0], s, rtol=1e-12, atol=1e-14)


# -------------------------------------------------------------- invariants
def test_retrieval_with_orthonormal_keys_returns_last_value():
    rng = np.random.default_rng(7)
    dk, dv, T = 8, 6, 40
    basis = np.linalg.qr(rng.standard_normal((dk, dk)))[0]   # orthonormal rows
    S0 = rng.standard_normal((1, 1, dk, dv))
    widx = rng.integers(0, dk, T)                 # which key is written at t
    qidx = rng.integers(0, dk, T)                 # which key is queried at t
    k = basis[widx][:, None, :]
    q = basis[qidx][:, None, :]
    v = rng.standard_normal((T, 1, dv))
    g = np.zeros((T, 1, dk))
    beta = np.ones((T, 1))
    z = np.full((T, 1, dv), 30.0)                # gate = sigmoid(30) ~ 1 - 9e-14
    out, final = oracle.forward(q, k, v, g, beta, z, init_state=S0)
    last = {i: S0[0, 0].T @ basis[i] for i in range(dk)}
    gate = 1.0 / (1.0 + math.exp(-30.0))
    for t in range(T):
        last[int(widx[t])] = v[t, 0]
        np.testing.assert_allclose(out[t, 0], gate * last[int(qidx[t])], rtol=0, atol=1e-12)
    for i in range(dk):
        np.testing.assert_allclose(final[0, 0].T @ basis[i], last[i], atol=1e-12)


def test_neg_inf_log_decay_resets_state():
    rng = np.random.default_rng(8)
    T, H, dk, dv, t0 = 20, 2, 5, 4, 7
    q, k, v, g, beta, z = random_inputs(rng, T, H, dk, dv)
    g[t0] = -np.inf
    S0 = rng.standard_normal((1, H, dk, dv))
    out, final = oracle.forward(q, k, v, g, beta, z, init_state=S0)
    sl = slice(t0, T)
    out2, final2 = oracle.forward(q[sl], k[sl], v[sl], g[sl], beta[sl], z[sl])
    np.testing.assert_array_equal(out[sl], out2)
    np.testing.assert_array_equal(final, final2)
    # and the earlier outputs did depend on S0
    out3, _ = oracle.forward(q, k, v, g, beta, z)
    assert np.max(np.abs(out3[:t0] - out[:t0])) > 1e-3


@pytest.mark.parametrize("chunk", [1, 3, 16, 64])
def test_chunkwise_form_equals_recurrence(chunk):
    rng = np.random.default_rng(100 + chunk)
    lens = [37, 0, 16, 5, 70]
    T, H, dk, dv = sum(lens), 2, 8, 6
    q, k, v, g, beta, z = random_inputs(rng, T, H, dk, dv)
    g[3, 0, 2] = -np.inf              # reset one channel of one head
    g[40:44, 1, :] = 0.0              # no-decay stretch
    g[50:, :, 1] = -5.0               # pinned at the floor
    cu = np.concatenate([[0], np.cumsum(lens)])
    S0 = rng.standard_normal((len(lens), H, dk, dv)) * 0.5
    ref_out, ref_fin = oracle.forward(q, k, v, g, beta, z, init_state=S0, cu_seqlens=cu, scale=0.9)
    out, fin = chunkwise.forward(q, k, v, g, beta, z, init_state=S0, cu_seqlens=cu, chunk=chunk,
                                 scale=0.9)
    assert rel_err(out, ref_out) < 1e-12
    assert rel_err(fin, ref_fin) < 1e-12


@pytest.mark.parametrize("tau", [32, 45])
def test_split_then_concat_equals_single_call(tau):
    rng = np.random.default_rng(9)
    T, H, dk, dv = 64, 2, 6, 5
    q, k, v, g, beta, z = random_inputs(rng, T, H, dk, dv)
    S0 = rng.standard_normal((1, H, dk, dv))
    full_out, full_fin = oracle.forward(q, k, v, g, beta, z, init_state=S0)
    a, b = slice(0, tau), slice(tau, T)
    o1, s1 = oracle.forward(q[a], k[a], v[a], g[a], beta[a], z[a], init_state=S0)
    o2, s2 = oracle.forward(q[b], k[b], v[b], g[b], beta[b], z[b], init_state=s1)
    np.testing.assert_array_equal(np.concatenate([o1, o2]), full_out)
    np.testing.assert_array_equal(s2, full_fin)
    # the chunkwise form agrees across an unaligned split too
    c1, t1 = chunkwise.forward(q[a], k[a], v[a], g[a], beta[a], z[a], init_state=S0, chunk=16)
    c2, t2 = chunkwise.forward(q[b], k[b], v[b], g[b], beta[b], z[b], init_state=t1, chunk=16)
    assert rel_err(np.concatenate([c1, c2]), full_out) < 1e-12
    assert rel_err(t2, full_fin) < 1e-12


def test_decode_steps_equal_forward():
    rng = np.random.default_rng(10)
    T, H, dk, dv, N = 11, 3, 4, 5, 2
    ins = [random_inputs(rng, T, H, dk, dv) for _ in range(N)]
    S0 = rng.standard_normal((N, H, dk, dv))
    state = S0.copy()
    ys = []
    for t in range(T):
        step = [np.stack([ins[n][i][t] for n in range(N)]) for i in range(6)]
        ys.append(oracle.decode_step(*step, state))
    for n in range(N):
        out, fin = oracle.forward(*ins[n], init_state=S0[n:n + 1])
        np.testing.assert_allclose(np.stack([y[n] for y in ys]), out, rtol=1e-14, atol=1e-15)
        np.testing.assert_allclose(state[n], fin[0], rtol=1e-14, atol=1e-15)


def test_linear_in_initial_state_and_values():
    rng = np.random.default_rng(12)
    T, H, dk, dv = 25, 2, 5, 4
    q, k, v1, g, beta, z = random_inputs(rng, T, H, dk, dv)
    v2 = rng.standard_normal(v1.shape)
    s1, s2 = rng.standard_normal((2, 1, H, dk, dv))
    al, be = 0.7, -1.3
    o1, f1 = oracle.forward(q, k, v1, g, beta, z, init_state=s1)
    o2, f2 = oracle.forward(q, k, v2, g, beta, z, init_state=s2)
    o3, f3 = oracle.forward(q, k, al * v1 + be * v2, g, beta, z, init_state=al * s1 + be * s2)
    assert rel_err(o3, al * o1 + be * o2) < 1e-12
    assert rel_err(f3, al * f1 + be * f2) < 1e-12


def test_value_columns_are_separable():
    rng = np.random.default_rng(13)
    T, H, dk, dv = 30, 2, 5, 8
    q, k, v, g, beta, z = random_inputs(rng, T, H, dk, dv)
    S0 = rng.standard_normal((1, H, dk, dv))
    out, fin = oracle.forward(q, k, v, g, beta, z, init_state=S0)
    perm = rng.permutation(dv)
    po, pf = oracle.forward(q, k, v[..., perm], g, beta, z[..., perm], init_state=S0[..., perm])
    np.testing.assert_array_equal(po, out[..., perm])
    np.testing.assert_array_equal(pf, fin[..., perm])
    lo, hi = slice(0, 3), slice(3, dv)
    ao, af = oracle.forward(q, k, v[..., lo], g, beta, z[..., lo], init_state=S0[..., lo])
    bo, bf = oracle.forward(q, k, v[..., hi], g, beta, z[..., hi], init_state=S0[..., hi])
    np.testing.assert_array_equal(np.concatenate([ao, bo], -1), out)
    np.testing.assert_array_equal(np.concatenate([af, bf], -1), fin)


def test_state_norm_bound_per_step():
    # unit keys, beta in [0, 1], g <= 0  =>  ||S_t||_F <= ||S_{t-1}||_F + beta_t ||v_t||
    rng = np.random.default_rng(14)
    T, H, dk, dv = 60, 2, 6, 4
    q, k, v, g, beta, z = random_inputs(rng, T, H, dk, dv, g_lo=-0.3)
    state = rng.standard_normal((1, H, dk, dv)) * 3
    for t in range(T):
        before = np.linalg.norm(state.reshape(H, -1), axis=1)
        oracle.decode_step(q[t:t + 1], k[t:t + 1], v[t:t + 1], g[t:t + 1], beta[t:t + 1],
                           z[t:t + 1], state)
        after = np.linalg.norm(state.reshape(H, -1), axis=1)
        bound = before + beta[t] * np.linalg.norm(v[t], axis=-1)
        assert np.all(after <= bound * (1 + 1e-12))


def test_float32_inputs_are_widened_exactly():
    rng = np.random.default_rng(15)
    T, H, dk, dv = 20, 2, 4, 4
    ins = [x.astype(np.float32) for x in random_inputs(rng, T, H, dk, dv)]
    o32, f32 = oracle.forward(*ins)
    o64, f64 = oracle.forward(*[x.astype(np.float64) for x in ins])
    np.testing.assert_array_equal(o32, o64)
    np.testing.assert_array_equal(f32, f64)


def test_argument_errors():
    rng = np.random.default_rng(16)
    q, k, v, g, beta, z = random_inputs(rng, 8, 1, 2, 2)
    with pytest.raises(ValueError):
        oracle.forward(q, k, v, g, beta, z, cu_seqlens=np.array([0, 5, 3, 8]))
    with pytest.raises(ValueError):
        oracle.forward(q, k, v, g, beta, z, init_state=np.zeros((2, 1, 2, 2)))


# ----------------------------------------------- streaming comparison (long inputs)
def _bf16_bits(x):
    """Round float64 values to bfloat16 with torch (nearest even) and return
    (the bit patterns as uint16, the same values as float32)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy(), t.float().numpy()


def test_compare_widens_bf16_exactly_and_tracks_per_unit_maxima():
    """bfloat16 bit patterns (rounded by torch, an independent library) widen
    to the very values forward() sees as float32, and err / ref are the
    per-(sequence, head) maxima numpy finds on forward()'s own output; an
    empty sequence reports 0 and keeps its initial state."""
    rng = np.random.default_rng(21)
    lens = [7, 0, 19]
    T, H, dk, dv = sum(lens), 3, 8, 6
    cu = np.concatenate([[0], np.cumsum(lens)])
    bits, vals = zip(*(_bf16_bits(x) for x in random_inputs(rng, T, H, dk, dv)))
    init = rng.standard_normal((len(lens), H, dk, dv)) * 0.1
    ref_out, ref_fin = oracle.forward(*vals, init_state=init, cu_seqlens=cu, scale=0.8)
    x_bits, x_vals = _bf16_bits(ref_out + rng.standard_normal(ref_out.shape) * 1e-3)
    err, ref, fin = oracle.forward_compare(*bits, x_bits, init_state=init, cu_seqlens=cu,
                                           scale=0.8, bf16=True)
    np.testing.assert_array_equal(fin, ref_fin)
    for n in range(len(lens)):
        sl = slice(cu[n], cu[n + 1])
        for h in range(H):
            d = np.abs(x_vals[sl, h].astype(np.float64) - ref_out[sl, h])
            assert err[n, h] == (d.max() if d.size else 0.0)
            assert ref[n, h] == (np.abs(ref_out[sl, h]).max() if d.size else 0.0)
    np.testing.assert_array_equal(fin[1], init[1])
    # float32 inputs and output give the same maxima as their values
    err32, ref32, _ = oracle.forward_compare(*vals, x_vals, init_state=init, cu_seqlens=cu,
                                             scale=0.8)
    np.testing.assert_array_equal(err32, err)
    np.testing.assert_array_equal(ref32, ref)


def test_compare_counts_nan_as_infinite_error():
    rng = np.random.default_rng(22)
    ins = [x.astype(np.float32) for x in random_inputs(rng, 12, 2, 4, 4)]
    out, _ = oracle.forward(*ins)
    x = out.astype(np.float32)
    x[5, 1, 2] = np.nan
    err, ref, _ = oracle.forward_compare(*ins, x)
    assert err[0, 1] == np.inf and np.isfinite(err[0, 0])
