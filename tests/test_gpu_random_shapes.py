"""GPU parity over seeded random shapes: the forward and the backward through
the C ABI against the fp64 oracle, on shapes drawn (with fixed seeds) from a
mix of chunk-edge lengths (0, 1, 15-17, 63-65, 127-129) and free lengths, head
counts that are and are not multiples of 8, fixed-length batches and packed
varlen sequences, zero and random initial states, final state requested or
not, and scales other than 1.  Each case prints its shape before it runs.
Tolerances are those of the other parity tests: 2e-2 (outputs, gradients) and
1e-2 (states) for bf16, 1e-4 for the fp32 path."""
from __future__ import annotations

import numpy as np
import pytest
import torch

from test_gpu_backward import cotangents, run_bf16_case, run_case
from test_gpu_parity import (TOL_BF16_OUT, TOL_BF16_STATE, TOL_F32, check, dev,  # noqa: F401
                             run_gpu, run_oracle, say, small_inputs)

pytestmark = pytest.mark.gpu

EDGES = (0, 1, 15, 16, 17, 63, 64, 65, 127, 128, 129)


def draw_case(seed, d, max_len):
    """(dtype, B, T, H, lengths or None, init_std, g_mode, scale, want_final)."""
    r = np.random.default_rng([7301, seed])
    H = int(r.choice([1, 2, 3, 5, 8, 12]))
    if r.random() < 0.6:
        n = int(r.integers(1, 6))
        lengths = [int(r.choice(EDGES)) if r.random() < 0.5 else int(r.integers(1, max_len))
                   for _ in range(n)]
        B, T = 1, 0
    else:
        lengths = None
        B = int(r.integers(1, 4))
        T = int(r.choice(EDGES[1:])) if r.random() < 0.5 else int(r.integers(1, max_len))
    init_std = float(r.choice([0.0, 0.02 if d == 128 else 0.3]))
    g_mode = str(r.choice(["random", "random", "slow", "zero", "pinned"]))
    scale = float(r.choice([1.0, 0.5, 0.125]))
    want_final = bool(r.random() < 0.8)
    return B, T, H, lengths, init_std, g_mode, scale, want_final


def label(seed, B, T, H, lengths, init_std, g_mode, scale, want_final):
    shape = f"lengths={lengths}" if lengths is not None else f"B={B} T={T}"
    return (f"seed {seed}: {shape} H={H} init_std={init_std} g={g_mode} scale={scale} "
            f"final={want_final}")


@pytest.mark.parametrize("dtype,d,seed", [(torch.bfloat16, 128, s) for s in range(20)] +
                                         [(torch.float32, 16, s) for s in range(8)])
def test_forward_random_shape(dev, dtype, d, seed):
    B, T, H, lengths, init_std, g_mode, scale, want_final = draw_case(
        seed, d, 700 if d == 128 else 200)
    name = f"{'bf16' if d == 128 else 'f32'} forward " + label(
        seed, B, T, H, lengths, init_std, g_mode, scale, want_final)
    say(name)
    x = small_inputs(dtype, B, T, H, d, d, 7400 + seed + 50 * d, lengths=lengths,
                     init_std=init_std, g_mode=g_mode)
    out, fin = run_gpu(x, dev, chunk=64 if d == 128 else 16, scale=scale,
                       output_final_state=want_final)
    ref_out, ref_fin = run_oracle(x, scale=scale)
    if not want_final:
        assert fin is None
    tol_out, tol_state = (TOL_BF16_OUT, TOL_BF16_STATE) if d == 128 else (TOL_F32, TOL_F32)
    check(out, fin, ref_out, ref_fin if want_final else None, tol_out, tol_state, name)


@pytest.mark.parametrize("dtype,d,seed", [(torch.bfloat16, 128, s) for s in range(8)] +
                                         [(torch.float32, 16, s) for s in range(4)])
def test_backward_random_shape(dev, dtype, d, seed):
    B, T, H, lengths, init_std, g_mode, scale, _ = draw_case(100 + seed, d, 300 if d == 128 else 150)
    name = label(100 + seed, B, T, H, lengths, init_std, g_mode, scale, True)
    say(f"{'bf16' if d == 128 else 'f32'} backward {name}")
    x = small_inputs(dtype, B, T, H, d, d, 7600 + seed + 50 * d, lengths=lengths,
                     init_std=init_std, g_mode=g_mode)
    dy, dfin = cotangents(x, 7700 + seed, 0.05 if d == 128 else 0.2)
    if d == 128:
        run_bf16_case(dev, x, dy, dfin, scale, name)
    else:
        run_case(dev, x, dy, dfin, scale, name, TOL_F32)


@pytest.mark.parametrize("dtype,d,seed", [(torch.bfloat16, 128, 0), (torch.float32, 16, 1),
                                         (torch.bfloat16, 16, 2), (torch.float32, 128, 3),
                                         (torch.bfloat16, 128, 4), (torch.bfloat16, 128, 5),
                                         (torch.float32, 128, 6), (torch.bfloat16, 16, 7)])
def test_decode_random_shape(dev, dtype, d, seed):
    """A few decode steps on a random (N, H) with random prologue bits, against
    the oracle's decode step (outputs and the state after every step)."""
    import numpy as np_

    import oracle
    from oracle import prologue as P
    from test_gpu_parity import np32, rel
    import kimi_delta_attention_chunkwise_amd as kda_

    r = np_.random.default_rng([7801, seed])
    N, H, steps = int(r.integers(1, 40)), int(r.choice([1, 3, 8, 13])), 3
    pro = int(r.choice([0, 1, 6, 7]))
    say(f"decode {dtype} d={d} seed {seed}: N={N} H={H} prologue={pro}, {steps} steps")
    gen = torch.Generator().manual_seed(7900 + seed)
    st = torch.randn(N, H, d, d, generator=gen) * 0.05
    ref = st.double().numpy().copy()
    state = st.to(dev)
    worst_o = worst_s = 0.0
    for t in range(steps):
        x = {key: torch.randn(*shape, generator=gen) for key, shape in
             (("q", (N, H, d)), ("k", (N, H, d)), ("v", (N, H, d)), ("g", (N, H, d)),
              ("beta", (N, H)), ("z", (N, H, d)))}
        if not pro & P.QK_L2NORM:
            x["q"] = x["q"] / x["q"].norm(dim=-1, keepdim=True)
            x["k"] = x["k"] / x["k"].norm(dim=-1, keepdim=True)
        if not pro & P.BETA_SIGMOID:
            x["beta"] = torch.sigmoid(x["beta"])
        if not pro & P.G_SOFTPLUS:
            x["g"] = torch.clamp(-torch.nn.functional.softplus(x["g"]), min=-5.0)
        x = {key: val.to(dtype) for key, val in x.items()}
        out = kda_.decode_step(*[x[key].to(dev) for key in ("q", "k", "v", "g", "beta", "z")],
                               state, prologue=pro)
        torch.cuda.synchronize()
        xs = {key: np32(val) for key, val in x.items()}
        q, k, beta, g = P.apply(xs["q"], xs["k"], xs["beta"], xs["g"], pro)
        ry = oracle.decode_step(q, k, xs["v"].astype(np_.float64), g, beta,
                                xs["z"].astype(np_.float64), ref)
        worst_o = max(worst_o, rel(np32(out), ry))
        worst_s = max(worst_s, rel(np32(state), ref))
    say(f"decode seed {seed}: worst out rel err {worst_o:.3e}, state {worst_s:.3e}")
    tol = TOL_BF16_OUT if dtype == torch.bfloat16 else 1e-5
    assert worst_o <= tol and worst_s <= 1e-4
