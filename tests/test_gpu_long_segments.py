"""GPU: a long single sequence, which runs in segments on two streams.

From 1,024 chunks on, ``kda_chunk_fwd`` over one sequence (no cu_seqlens, no
snapshots, a final state wanted) runs in segments of at least 512 chunks,
handing the fp32 state from segment to segment.  Up to 32 heads it is
pipelined: the caller's stream prepares segment by segment and runs finished
segments' outputs, and a second stream runs each segment's chain (on
workgroups of four value blocks) beside the next preparation.  With more
heads the whole preparation runs first and each segment's chain (one value
block per workgroup) on the second stream, the outputs beside it.  The state
passes through memory unchanged, so either way the result must be bitwise
that of calls too short to be segmented, chained by hand, or of the same
sequence given through cu_seqlens (which keeps one stream); and it must match
the oracle.
"""
from __future__ import annotations

import pytest
import torch

import kimi_delta_attention_chunkwise_amd as kda

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
    print(f"[gpu-long-segments] {msg}", flush=True)


def test_segmented_chain_equals_short_calls_and_oracle(dev):
    T, H, cut = 70_000, 2, 32_768          # 1,094 chunks: segments of 512, 512 and 70
    say(f"B=1 H={H} T={T}: one call against two calls of {cut} and {T - cut} tokens")
    x = small_inputs(torch.bfloat16, 1, T, H, 128, 128, 77, init_std=0.02)
    xd = to(x, dev)
    out, fin = kda.chunk_fwd(*[xd[k] for k in KEYS], init_state=xd["init_state"])
    a = [xd[k][:, :cut].contiguous() for k in KEYS]
    b = [xd[k][:, cut:].contiguous() for k in KEYS]
    o1, s1 = kda.chunk_fwd(*a, init_state=xd["init_state"])
    o2, s2 = kda.chunk_fwd(*b, init_state=s1)
    torch.cuda.synchronize()
    assert torch.equal(out, torch.cat([o1, o2], dim=1)), "outputs differ from the short calls"
    assert torch.equal(fin, s2), "final state differs from the short calls"
    # the same call with the final state written over the initial state
    st = xd["init_state"].clone()
    out3, _ = kda.chunk_fwd(*[xd[k] for k in KEYS], init_state=st, final_state=st)
    torch.cuda.synchronize()
    assert torch.equal(out3, out) and torch.equal(st, fin), "in-place state differs"
    say("oracle comparison, both heads over all tokens")
    ro, rf = run_oracle(x)
    check(out, fin, ro, rf, 2e-2, 1e-2, f"long segments T={T}")


def test_segmented_calls_from_two_threads(dev):
    """Two host threads, each on its own stream, run segmented forwards at the
    same time (they share the library's second stream and its events): each
    result must be bitwise that of the same call made alone."""
    import threading

    T, H = 66_000, 2                       # 1,032 chunks: two segments
    say(f"two threads, B=1 H={H} T={T} each, on two streams")
    xs = [to(small_inputs(torch.bfloat16, 1, T, H, 128, 128, 78 + i, init_std=0.02), dev)
          for i in range(2)]
    alone = []
    for x in xs:
        alone.append(kda.chunk_fwd(*[x[k] for k in KEYS], init_state=x["init_state"]))
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(device=dev) for _ in xs]   # default priority
    results = [None, None]
    errors = []

    def work(i):
        try:
            with torch.cuda.stream(streams[i]):
                got = []
                for _ in range(3):
                    x = xs[i]
                    got.append(kda.chunk_fwd(*[x[k] for k in KEYS], init_state=x["init_state"]))
                results[i] = got
        except Exception as exc:  # reported below, in the main thread
            errors.append(exc)

    threads = [threading.Thread(target=work, args=(i,)) for i in range(2)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    torch.cuda.synchronize()
    assert not errors, errors
    for i in range(2):
        for out, fin in results[i]:
            assert torch.equal(out, alone[i][0]) and torch.equal(fin, alone[i][1]), (
                f"thread {i}: result differs from the call made alone")


def test_long_forward_captured_in_a_graph(dev):
    """A forward long enough for the segmented schedule, captured in a HIP
    graph: while the caller's stream is capturing, the library keeps every
    kernel on that stream (no work of its shared second stream enters the
    capture).  Each replay, with eager library work and synchronisations in
    between, must be bitwise the eager call; the result matches the oracle."""
    T, H = 70_000, 2
    say(f"graph capture of B=1 H={H} T={T}, three replays")
    x = small_inputs(torch.bfloat16, 1, T, H, 128, 128, 79, init_std=0.02)
    xd = to(x, dev)
    ins = [xd[k] for k in KEYS]
    ref_out, ref_fin = kda.chunk_fwd(*ins, init_state=xd["init_state"])
    ws = torch.empty(kda.chunk_fwd_workspace_bytes(1, T, 1, H, 128, 128, 64, torch.bfloat16,
                                                   False), dtype=torch.uint8, device=dev)
    out = torch.empty_like(ref_out)
    fin = torch.empty_like(ref_fin)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        kda.chunk_fwd(*ins, init_state=xd["init_state"], workspace=ws, out=out, final_state=fin)
    other = to(small_inputs(torch.bfloat16, 1, T, H, 128, 128, 80, init_std=0.02), dev)
    for rep in range(3):
        out.fill_(0)
        fin.fill_(0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref_out) and torch.equal(fin, ref_fin), f"replay {rep} differs"
        # eager work of the library between replays (the segmented schedule)
        kda.chunk_fwd(*[other[k] for k in KEYS], init_state=other["init_state"])
        torch.cuda.synchronize()
    ro, rf = run_oracle(x)
    check(out, fin, ro, rf, 2e-2, 1e-2, f"graph-captured long forward T={T}")


LONG_CASES = {
    # name: (H, prologue bits, per-chunk records)
    "pipelined_with_prologue": (2, kda.PRO_QK_L2NORM | kda.PRO_BETA_SIGMOID | kda.PRO_G_SOFTPLUS,
                                False),
    "pipelined_per_chunk_records": (2, 0, True),
    "prep_first_40_heads": (40, 0, False),     # the chain would need more than a quarter of the CUs
}


@pytest.mark.parametrize("case", list(LONG_CASES))
def test_segmented_schedules_equal_one_stream(dev, case):
    """Each segmented schedule against the same sequence given through
    cu_seqlens = [0, T], which keeps every kernel on one stream: bitwise."""
    H, pro, per_chunk = LONG_CASES[case]
    T = 66_000
    say(f"{case}: B=1 H={H} T={T} prologue={pro} chunk_records={per_chunk}")
    xd = to(small_inputs(torch.bfloat16, 1, T, H, 128, 128, 79, init_std=0.02), dev)
    args = [xd[k] for k in KEYS]
    out, fin = kda.chunk_fwd(*args, init_state=xd["init_state"], prologue=pro,
                             chunk_records=per_chunk)
    cu = torch.tensor([0, T], dtype=torch.int32, device=dev)
    ro, rf = kda.chunk_fwd(*args, init_state=xd["init_state"], cu_seqlens=cu, prologue=pro,
                           chunk_records=per_chunk)
    torch.cuda.synchronize()
    assert torch.equal(out, ro), f"{case}: outputs differ from the one-stream call"
    assert torch.equal(fin, rf), f"{case}: final state differs from the one-stream call"
