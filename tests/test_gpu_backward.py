"""GPU parity of the chunkwise backward (kda_chunk_bwd through the C ABI)
against the oracle's backward: the gradients of
sum(dY * Y) + sum(dS_final * S_final) with respect to every input, on the same
seeded tensors.  Error per gradient tensor: max|x - ref| / max|ref|; the fp32
path's tolerance is 1e-4, as for its forward."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import kimi_delta_attention_chunkwise_amd as kda
import oracle
import workloads as W
from test_gpu_parity import TOL_F32, dev, np32, rel, say, small_inputs, to  # noqa: F401

pytestmark = pytest.mark.gpu

GRADS = (("q", "dq"), ("k", "dk"), ("v", "dv"), ("g", "dg"), ("beta", "dbeta"), ("gate", "dz"))


def cotangents(x, seed, dfinal_std):
    """dY ~ N(0, 1) like the output; dS_final ~ dfinal_std N(0, 1) or None."""
    gen = torch.Generator().manual_seed(seed)
    dy = torch.randn(x["v"].shape, generator=gen).to(x["v"].dtype)
    N = x["cu_seqlens"].numel() - 1 if x.get("cu_seqlens") is not None else x["q"].shape[0]
    H, dk, dv = x["q"].shape[2], x["q"].shape[3], x["v"].shape[3]
    dfin = torch.randn(N, H, dk, dv, generator=gen) * dfinal_std if dfinal_std else None
    return dy, dfin


def run_case(dev, x, dy, dfin, scale, label, tol):
    xd = to(x, dev)
    gr = kda.chunk_bwd(xd["q"], xd["k"], xd["v"], xd["g"], xd["beta"], xd["z"], dy.to(dev),
                       init_state=xd.get("init_state"),
                       grad_final_state=None if dfin is None else dfin.to(dev),
                       cu_seqlens=xd.get("cu_seqlens"), scale=scale)
    torch.cuda.synchronize()
    cu = x.get("cu_seqlens")
    ref = oracle.backward(np32(x["q"]), np32(x["k"]), np32(x["v"]), np32(x["g"]),
                          np32(x["beta"]), np32(x["z"]), np32(dy),
                          init_state=np32(x.get("init_state")), dfinal=np32(dfin),
                          cu_seqlens=None if cu is None else cu.numpy(), scale=scale)
    errs = {name: rel(np32(gr[name]), ref[key]) for name, key in GRADS}
    errs["init_state"] = rel(np32(gr["init_state"]), ref["dinit"])
    say(f"backward {label}: " + ", ".join(f"d{k} {e:.2e}" for k, e in errs.items()))
    for name, _ in GRADS:
        assert np.all(np.isfinite(np32(gr[name]))), f"{label}: non-finite d{name}"
    bad = {k: e for k, e in errs.items() if e > tol}
    assert not bad, f"{label}: gradient errors above {tol}: {bad}"


def test_tiny_f32_workload_backward(dev):
    w = W.WORKLOADS["tiny_f32"]
    say("backward tiny_f32 B=1 H=2 T=64 dk=dv=16 chunk=16")
    x = W.prefill_inputs(w, seed=0)
    dy, dfin = cotangents(x, 500, 0.0)
    run_case(dev, x, dy, dfin, 1.0, "tiny_f32", TOL_F32)


@pytest.mark.parametrize("case", ["varlen_init", "ragged_batch", "floor_decay", "zero_decay",
                                  "long"])
def test_f32_backward_cases(dev, case):
    say(f"backward f32 case {case}")
    f32 = torch.float32
    if case == "varlen_init":
        x = small_inputs(f32, 1, 0, 3, 16, 16, 21, lengths=[0, 5, 16, 37, 1, 0, 33],
                         init_std=0.5)
    elif case == "ragged_batch":
        x = small_inputs(f32, 3, 45, 2, 16, 16, 22, init_std=0.3)
    elif case == "floor_decay":
        # every log-decay at the -5 floor: G spans -80 inside a chunk
        x = small_inputs(f32, 2, 40, 2, 16, 16, 23, init_std=0.3)
        x["g"] = torch.full_like(x["g"], -5.0)
    elif case == "zero_decay":
        x = small_inputs(f32, 1, 50, 2, 16, 16, 24, init_std=0.3, g_mode="zero")
    else:
        x = small_inputs(f32, 2, 1000, 4, 16, 16, 25, init_std=0.1)
    dy, dfin = cotangents(x, 600, 0.2)
    run_case(dev, x, dy, dfin, 0.75, case, TOL_F32)


def test_f32_backward_empty(dev):
    """T = 0: no token gradients, and the initial-state gradient is dS_final."""
    x = small_inputs(torch.float32, 2, 0, 2, 16, 16, 26, init_std=0.3)
    dy, dfin = cotangents(x, 700, 0.5)
    xd = to(x, dev)
    gr = kda.chunk_bwd(xd["q"], xd["k"], xd["v"], xd["g"], xd["beta"], xd["z"], dy.to(dev),
                       init_state=xd["init_state"], grad_final_state=dfin.to(dev))
    torch.cuda.synchronize()
    assert gr["q"].numel() == 0
    assert torch.equal(gr["init_state"].cpu(), dfin)


# ------------------------------------------------------------------ bf16 path
# Gradients are outputs of the backward and the initial-state gradient is a
# state: the bf16 tolerances of the forward (2e-2 on outputs, 1e-2 on states)
# apply to them.
TOL_BF16_GRAD, TOL_BF16_DSTATE = 2e-2, 1e-2


def run_bf16_case(dev, x, dy, dfin, scale, label):
    xd = to(x, dev)
    gr = kda.chunk_bwd(xd["q"], xd["k"], xd["v"], xd["g"], xd["beta"], xd["z"], dy.to(dev),
                       init_state=xd.get("init_state"),
                       grad_final_state=None if dfin is None else dfin.to(dev),
                       cu_seqlens=xd.get("cu_seqlens"), scale=scale)
    torch.cuda.synchronize()
    cu = x.get("cu_seqlens")
    ref = oracle.backward(np32(x["q"]), np32(x["k"]), np32(x["v"]), np32(x["g"]),
                          np32(x["beta"]), np32(x["z"]), np32(dy),
                          init_state=np32(x.get("init_state")), dfinal=np32(dfin),
                          cu_seqlens=None if cu is None else cu.numpy(), scale=scale)
    errs = {name: rel(np32(gr[name]), ref[key]) for name, key in GRADS}
    es = rel(np32(gr["init_state"]), ref["dinit"])
    say(f"backward bf16 {label}: " + ", ".join(f"d{k} {e:.2e}" for k, e in errs.items()) +
        f", dinit {es:.2e}")
    for name, _ in GRADS:
        assert np.all(np.isfinite(np32(gr[name]))), f"{label}: non-finite d{name}"
    bad = {k: e for k, e in errs.items() if e > TOL_BF16_GRAD}
    assert not bad, f"{label}: gradient errors above {TOL_BF16_GRAD}: {bad}"
    assert es <= TOL_BF16_DSTATE, f"{label}: initial-state gradient error {es}"


@pytest.mark.parametrize("case", ["ragged_batch", "varlen_edges", "pinned_floor", "floor_decay",
                                  "zero_decay"])
def test_bf16_backward_cases(dev, case):
    say(f"backward bf16 case {case}")
    bf = torch.bfloat16
    if case == "ragged_batch":
        x = small_inputs(bf, 2, 200, 2, 128, 128, 31, init_std=0.02)
    elif case == "varlen_edges":
        x = small_inputs(bf, 1, 0, 3, 128, 128, 32, lengths=[0, 1, 15, 17, 63, 64, 65, 129, 0],
                         init_std=0.02)
    elif case == "pinned_floor":
        x = small_inputs(bf, 1, 300, 2, 128, 128, 33, init_std=0.02, g_mode="pinned")
    elif case == "floor_decay":
        x = small_inputs(bf, 1, 150, 2, 128, 128, 34, init_std=0.02)
        x["g"] = torch.full_like(x["g"], -5.0)
    else:
        x = small_inputs(bf, 1, 130, 2, 128, 128, 35, init_std=0.02, g_mode="zero")
    dy, dfin = cotangents(x, 800, 0.05)
    run_bf16_case(dev, x, dy, dfin, 0.5 if case == "varlen_edges" else 1.0, case)


def test_bf16_backward_prefill_t4096_h8(dev):
    """The prefill workload's shape (B=1, H=8, T=4096, dk=dv=128), compared in full."""
    w = W.WORKLOADS["prefill_t4096_h8"]
    say("backward bf16 prefill_t4096_h8 B=1 H=8 T=4096")
    x = W.prefill_inputs(w, seed=0)
    dy, dfin = cotangents(x, 900, 0.05)
    run_bf16_case(dev, x, dy, dfin, 1.0, "prefill_t4096_h8")


def test_bf16_backward_reusing_forward_records(dev):
    """kda_chunk_bwd_ex on the workspace of a forward that kept per-chunk
    records (KDA_FWD_CHUNK_RECORDS): the same gradients bit for bit as the
    backward alone, and within tolerance of the oracle; the forward's outputs
    equal those of the default forward (pair records) within its tolerance."""
    say("backward bf16 reusing the forward's records (varlen, init state)")
    x = small_inputs(torch.bfloat16, 1, 0, 2, 128, 128, 36, lengths=[70, 0, 200, 64, 5],
                     init_std=0.02)
    dy, dfin = cotangents(x, 901, 0.05)
    xd = to(x, dev)
    ws_f = torch.empty(kda.chunk_fwd_workspace_bytes(1, int(x["q"].shape[1]), 5, 2, 128, 128, 64,
                                                     torch.bfloat16, True, chunk_records=True),
                       dtype=torch.uint8, device=dev)
    out_c, fin_c = kda.chunk_fwd(xd["q"], xd["k"], xd["v"], xd["g"], xd["beta"], xd["z"],
                                 init_state=xd["init_state"], cu_seqlens=xd["cu_seqlens"],
                                 workspace=ws_f, scale=0.5, chunk_records=True)
    out_p, fin_p = kda.chunk_fwd(xd["q"], xd["k"], xd["v"], xd["g"], xd["beta"], xd["z"],
                                 init_state=xd["init_state"], cu_seqlens=xd["cu_seqlens"],
                                 scale=0.5)
    torch.cuda.synchronize()
    ro, rf = oracle.forward(*(np32(x[k]) for k in ("q", "k", "v", "g", "beta", "z")),
                            init_state=np32(x["init_state"]),
                            cu_seqlens=x["cu_seqlens"].numpy(), scale=0.5)
    for label, (o, f) in (("chunk records", (out_c, fin_c)), ("pair records", (out_p, fin_p))):
        eo, es = rel(np32(o), ro), rel(np32(f), rf)
        say(f"forward with {label}: out rel err {eo:.3e}, state rel err {es:.3e}")
        assert eo <= 2e-2 and es <= 1e-2
    kw = dict(init_state=xd["init_state"], grad_final_state=dfin.to(dev),
              cu_seqlens=xd["cu_seqlens"], scale=0.5)
    reused = kda.chunk_bwd(xd["q"], xd["k"], xd["v"], xd["g"], xd["beta"], xd["z"], dy.to(dev),
                           fwd_workspace=ws_f, **kw)
    alone = kda.chunk_bwd(xd["q"], xd["k"], xd["v"], xd["g"], xd["beta"], xd["z"], dy.to(dev),
                          **kw)
    torch.cuda.synchronize()
    for key in ("q", "k", "v", "g", "beta", "gate", "init_state"):
        assert torch.equal(reused[key], alone[key]), f"d{key} differs with reused records"
    run_bf16_case(dev, x, dy, dfin, 0.5, "reused records")


def test_bf16_backward_varlen_4seq_h32_full(dev):
    """The packed varlen workload at full size (4 sequences, lengths up to 32K, H=32,
    non-zero initial state), every gradient against the oracle's backward."""
    w = W.WORKLOADS["varlen_4seq_h32"]
    say(f"backward bf16 varlen_4seq_h32: lengths {W.varlen_lengths(w, 0)}")
    x = W.prefill_inputs(w, seed=0)
    dy, dfin = cotangents(x, 902, 0.02)
    run_bf16_case(dev, x, dy, dfin, 1.0, "varlen_4seq_h32")
