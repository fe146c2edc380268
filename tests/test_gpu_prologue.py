"""GPU parity of the fused input prologue (q/k L2 norm, beta = sigmoid(logit),
g = max(-5, -softplus(x))) against the oracle: the raw inputs go through
oracle/prologue.py in fp64 and then through the fp64 recurrence; the GPU gets
the same raw tensors and the prologue bits."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import kimi_delta_attention_chunkwise_amd as kda
import oracle
from oracle import prologue as P
from test_gpu_parity import (TOL_BF16_OUT, TOL_BF16_STATE, TOL_F32, dev, np32, rel, say,  # noqa: F401
                             to)

pytestmark = pytest.mark.gpu

ALL = kda.PRO_QK_L2NORM | kda.PRO_BETA_SIGMOID | kda.PRO_G_SOFTPLUS


def raw_inputs(dtype, tok_shape, H, dk, dv, seed, flags, lengths=None, init_std=0.0):
    """Raw projections: q, k ~ 3 N(0, 1) (not normalised), beta logits ~ N(0, 1),
    g pre-activations ~ 2 N(0, 1) (so the -5 floor is hit); inputs a flag does
    not cover are drawn prepared, as the recurrence needs them."""
    gen = torch.Generator().manual_seed(seed)
    n = lambda *s: torch.randn(*s, generator=gen)
    q, k = n(*tok_shape, H, dk) * 3.0, n(*tok_shape, H, dk) * 3.0
    if not flags & P.QK_L2NORM:
        q = q / q.norm(dim=-1, keepdim=True)
        k = k / k.norm(dim=-1, keepdim=True)
    beta = n(*tok_shape, H)
    if not flags & P.BETA_SIGMOID:
        beta = torch.sigmoid(beta)
    g = n(*tok_shape, H, dk) * 2.0
    if not flags & P.G_SOFTPLUS:
        g = torch.clamp(-torch.nn.functional.softplus(g), min=-5.0)
    d = {"q": q, "k": k, "v": n(*tok_shape, H, dv), "g": g, "beta": beta,
         "z": n(*tok_shape, H, dv)}
    d = {key: val.to(dtype) for key, val in d.items()}
    if lengths is not None:
        d["cu_seqlens"] = torch.tensor(np.concatenate([[0], np.cumsum(lengths)]),
                                       dtype=torch.int32)
        N = len(lengths)
    else:
        d["cu_seqlens"] = None
        N = tok_shape[0]
    d["init_state"] = (n(N, H, dk, dv) * init_std) if init_std else None
    return d


def oracle_prologue_forward(x, flags):
    q, k, beta, g = P.apply(np32(x["q"]), np32(x["k"]), np32(x["beta"]), np32(x["g"]), flags)
    cu = x.get("cu_seqlens")
    return oracle.forward(q, k, np32(x["v"]).astype(np.float64), g, beta,
                          np32(x["z"]).astype(np.float64), init_state=np32(x.get("init_state")),
                          cu_seqlens=None if cu is None else cu.numpy())


@pytest.mark.parametrize("flags", [P.QK_L2NORM, P.BETA_SIGMOID, P.G_SOFTPLUS, ALL])
def test_bf16_prologue_flags(dev, flags):
    x = raw_inputs(torch.bfloat16, (2, 300), 2, 128, 128, 60 + flags, flags, init_std=0.02)
    xd = to(x, dev)
    out, fin = kda.chunk_fwd(xd["q"], xd["k"], xd["v"], xd["g"], xd["beta"], xd["z"],
                             init_state=xd["init_state"], prologue=flags)
    torch.cuda.synchronize()
    ro, rf = oracle_prologue_forward(x, flags)
    eo, es = rel(np32(out), ro), rel(np32(fin), rf)
    say(f"bf16 prologue {flags}: out rel err {eo:.3e}, state rel err {es:.3e}")
    assert np.all(np.isfinite(np32(out)))
    assert eo <= TOL_BF16_OUT and es <= TOL_BF16_STATE


def test_bf16_prologue_varlen_snapshots(dev):
    lengths = [200, 0, 64, 333]
    x = raw_inputs(torch.bfloat16, (1, sum(lengths)), 2, 128, 128, 70, ALL, lengths=lengths,
                   init_std=0.02)
    xd = to(x, dev)
    out, fin, snaps = kda.chunk_fwd_snapshots(xd["q"], xd["k"], xd["v"], xd["g"], xd["beta"],
                                              xd["z"], 64, init_state=xd["init_state"],
                                              cu_seqlens=xd["cu_seqlens"], prologue=ALL)
    torch.cuda.synchronize()
    ro, rf = oracle_prologue_forward(x, ALL)
    eo, es = rel(np32(out), ro), rel(np32(fin), rf)
    say(f"bf16 prologue varlen: out rel err {eo:.3e}, state rel err {es:.3e}")
    assert eo <= TOL_BF16_OUT and es <= TOL_BF16_STATE
    # one snapshot: sequence 3 after 192 tokens equals the oracle's prefix state
    idx = {(n, t): s for n, t, s in kda.snapshot_index(lengths, 64, True)}
    a = int(x["cu_seqlens"][3])
    pre = {key: x[key][:, a:a + 192] for key in ("q", "k", "v", "g", "beta", "z")}
    pre["cu_seqlens"] = None
    pre["init_state"] = x["init_state"][3:4]
    _, rs = oracle_prologue_forward(pre, ALL)
    assert rel(np32(snaps[idx[(3, 192)]]), rs[0]) <= TOL_BF16_STATE


def test_f32_prologue(dev):
    x = raw_inputs(torch.float32, (2, 80), 2, 16, 16, 71, ALL, init_std=0.3)
    xd = to(x, dev)
    out, fin = kda.chunk_fwd(xd["q"], xd["k"], xd["v"], xd["g"], xd["beta"], xd["z"],
                             init_state=xd["init_state"], prologue=ALL)
    torch.cuda.synchronize()
    ro, rf = oracle_prologue_forward(x, ALL)
    eo, es = rel(np32(out), ro), rel(np32(fin), rf)
    say(f"f32 prologue: out rel err {eo:.3e}, state rel err {es:.3e}")
    assert eo <= TOL_F32 and es <= TOL_F32


@pytest.mark.parametrize("dtype,d,tol", [(torch.float32, 16, 1e-5), (torch.bfloat16, 128, 1e-4)])
def test_decode_prologue(dev, dtype, d, tol):
    N, H, steps = 5, 3, 12
    gen = torch.Generator().manual_seed(72)
    st0 = torch.randn(N, H, d, d, generator=gen) * 0.05
    state = st0.to(dev)
    ref = st0.double().numpy().copy()
    worst = 0.0
    for s in range(steps):
        x = raw_inputs(dtype, (N,), H, d, d, 100 + s, ALL)
        xd = to(x, dev)
        y = kda.decode_step(xd["q"], xd["k"], xd["v"], xd["g"], xd["beta"], xd["z"], state,
                            prologue=ALL)
        q, k, beta, g = P.apply(np32(x["q"]), np32(x["k"]), np32(x["beta"]), np32(x["g"]), ALL)
        ry = oracle.decode_step(q, k, np32(x["v"]).astype(np.float64), g, beta,
                                np32(x["z"]).astype(np.float64), ref)
        torch.cuda.synchronize()
        worst = max(worst, rel(np32(y), ry))
    es = rel(np32(state), ref)
    say(f"decode prologue {dtype} d={d}: worst out rel err {worst:.3e}, state rel err {es:.3e}")
    assert es <= tol
    assert worst <= (TOL_BF16_OUT if dtype == torch.bfloat16 else tol)
