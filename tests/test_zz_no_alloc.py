"""GPU: kda_chunk_fwd_noalloc, the forward that allocates nothing.

It runs the kernels of kda_chunk_fwd with the library's static per-GPU scratch
array as the workspace, so its results must be bitwise those of kda_chunk_fwd
on the same inputs.  Checked on two calls in a row, the second smaller than
the first (the array keeps the first call's contents), on a packed varlen
call with an initial state, under HIP graph capture with several replays, and
for the size limit.
"""
from __future__ import annotations

import pytest
import torch

import kimi_delta_attention_chunkwise_amd as kda
import workloads as W

from test_gpu_parity import check, run_oracle, small_inputs, to

pytestmark = pytest.mark.gpu
KEYS = ("q", "k", "v", "g", "beta", "z")


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no HIP device")
    kda.load_library()
    return torch.device("cuda:0")


def say(msg):
    print(f"[gpu-no-alloc] {msg}", flush=True)


def both(x, **kw):
    ins = [x[k] for k in KEYS]
    a = kda.chunk_fwd(*ins, init_state=x.get("init_state"), cu_seqlens=x.get("cu_seqlens"), **kw)
    b = kda.chunk_fwd_noalloc(*ins, init_state=x.get("init_state"),
                              cu_seqlens=x.get("cu_seqlens"), **kw)
    torch.cuda.synchronize()
    return a, b


def test_noalloc_equals_chunk_fwd_on_two_calls(dev):
    w = W.WORKLOADS["prefill_t4096_h8"]
    say("call 1: prefill_t4096_h8 (B=1, H=8, T=4096), bitwise against kda_chunk_fwd")
    x = W.prefill_inputs(w, device=dev, seed=3)
    (o1, f1), (o2, f2) = both(x)
    assert torch.equal(o1, o2) and torch.equal(f1, f2)
    say("call 2, smaller: varlen [0, 1, 63, 65, 129, 300] x 3 heads with an initial state")
    y = small_inputs(torch.bfloat16, 1, 0, 3, 128, 128, 90, lengths=[0, 1, 63, 65, 129, 300],
                     init_std=0.02)
    yd = to(y, dev)
    (o1, f1), (o2, f2) = both(yd)
    assert torch.equal(o1, o2) and torch.equal(f1, f2)
    ro, rf = run_oracle(y)
    check(o2, f2, ro, rf, 2e-2, 1e-2, "noalloc varlen")
    say("call 3: fp32 path (needs no scratch)")
    t = W.prefill_inputs(W.WORKLOADS["tiny_f32"], device=dev, seed=0)
    (o1, f1), (o2, f2) = both(t, chunk=16)
    assert torch.equal(o1, o2) and torch.equal(f1, f2)


def test_noalloc_under_graph_capture(dev):
    say("graph capture of kda_chunk_fwd_noalloc (B=2, T=300, H=4), three replays")
    x = to(small_inputs(torch.bfloat16, 2, 300, 4, 128, 128, 91, init_std=0.02), dev)
    ins = [x[k] for k in KEYS]
    ref_out, ref_fin = kda.chunk_fwd(*ins, init_state=x["init_state"])
    out, fin = torch.empty_like(ref_out), torch.empty_like(ref_fin)
    kda.chunk_fwd_noalloc(*ins, init_state=x["init_state"], out=out, final_state=fin)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        kda.chunk_fwd_noalloc(*ins, init_state=x["init_state"], out=out, final_state=fin)
    other = to(small_inputs(torch.bfloat16, 1, 500, 2, 128, 128, 92), dev)
    for rep in range(3):
        out.fill_(0)
        fin.fill_(0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref_out) and torch.equal(fin, ref_fin), f"replay {rep}"
        # eager use of the same scratch array between replays
        kda.chunk_fwd_noalloc(*[other[k] for k in KEYS])
        torch.cuda.synchronize()


def test_noalloc_size_limit(dev):
    rec = kda.chunk_fwd_workspace_bytes(1, 128, 1, 1, 128, 128, 64, torch.bfloat16, False)
    T = (kda.NOALLOC_SCRATCH_BYTES // rec) * 128 + 1        # one token past the limit, H = 1
    assert kda.chunk_fwd_workspace_bytes(1, T, 1, 1, 128, 128, 64, torch.bfloat16,
                                         False) > kda.NOALLOC_SCRATCH_BYTES
    say(f"T={T}, H=1: beyond the scratch array, refused before launch")
    x = to(small_inputs(torch.bfloat16, 1, T, 1, 128, 128, 93), dev)
    out = torch.full_like(x["v"], 3.0)
    with pytest.raises(kda.KdaError, match="KDA_ERR_SCRATCH_LIMIT"):
        kda.chunk_fwd_noalloc(*[x[k] for k in KEYS], out=out)
    torch.cuda.synchronize()
    assert torch.all(out == 3.0)
