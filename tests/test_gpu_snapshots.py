"""GPU parity of state snapshots (kda_chunk_fwd_snapshots) against the oracle.

A snapshot is the fp32 state after the first m * interval tokens of a
sequence.  The oracle's state at that point is its final state over that
prefix, computed segment by segment (each segment starts from the previous
segment's final state).  Checked: every written slot against the oracle, the
slots that match no snapshot left untouched, outputs and final states equal
to kda_chunk_fwd's bit for bit, and replay from a snapshot equal to the
single call bit for bit (the replay starts on a chunk boundary, so the
arithmetic is the same).
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import kimi_delta_attention_chunkwise_amd as kda
import oracle
from test_gpu_parity import TOL_BF16_STATE, TOL_F32, dev, np32, rel, say, small_inputs, to  # noqa: F401

pytestmark = pytest.mark.gpu

KEYS = ("q", "k", "v", "g", "beta", "z")


def seq_tokens(x, n):
    """Per-sequence token slices [1, len, ...] of input dict x."""
    cu = x.get("cu_seqlens")
    if cu is None:
        return {k: x[k][n:n + 1] for k in KEYS}
    a, b = int(cu[n]), int(cu[n + 1])
    return {k: x[k][:, a:b] for k in KEYS}


def oracle_prefix_states(x, n, interval, length):
    """Oracle states after m * interval tokens of sequence n, m = 1, 2, ..."""
    xs = seq_tokens(x, n)
    init = x.get("init_state")
    st = None if init is None else np32(init[n:n + 1])
    states = []
    for m in range(1, length // interval + 1):
        seg = {k: np32(xs[k][:, (m - 1) * interval:m * interval]) for k in KEYS}
        _, st = oracle.forward(seg["q"], seg["k"], seg["v"], seg["g"], seg["beta"], seg["z"],
                               init_state=st)
        states.append(st[0])
    return states


def run_snap(x, dev, interval):
    xd = to(x, dev)
    out, fin, snaps = kda.chunk_fwd_snapshots(xd["q"], xd["k"], xd["v"], xd["g"], xd["beta"],
                                              xd["z"], interval,
                                              init_state=xd.get("init_state"),
                                              cu_seqlens=xd.get("cu_seqlens"),
                                              snapshots=None)
    return xd, out, fin, snaps


def check_case(x, dev, interval, lengths, varlen, T, tol):
    xd = to(x, dev)
    B, Tt, H = xd["q"].shape[:3]
    N = len(lengths)
    slots = kda.snapshot_slots(B, Tt, N, 64 if xd["q"].dtype == torch.bfloat16 else 16,
                               interval, varlen)
    sentinel = torch.full((slots, H, xd["q"].shape[3], xd["v"].shape[3]), float("nan"),
                          device=dev)
    out, fin, snaps = kda.chunk_fwd_snapshots(xd["q"], xd["k"], xd["v"], xd["g"], xd["beta"],
                                              xd["z"], interval,
                                              init_state=xd.get("init_state"),
                                              cu_seqlens=xd.get("cu_seqlens"),
                                              snapshots=sentinel)
    # an interval that is an odd multiple of 64 splits a pair of chunks: that
    # call keeps per-chunk records, and so must the call it is compared with
    per_chunk = xd["q"].dtype == torch.bfloat16 and interval % 128 != 0
    out0, fin0 = kda.chunk_fwd(xd["q"], xd["k"], xd["v"], xd["g"], xd["beta"], xd["z"],
                               init_state=xd.get("init_state"), cu_seqlens=xd.get("cu_seqlens"),
                               chunk_records=per_chunk)
    torch.cuda.synchronize()
    assert torch.equal(out, out0) and torch.equal(fin, fin0), "snapshots changed the result"
    snaps = snaps.cpu()
    index = kda.snapshot_index(lengths, interval, varlen, T)
    written = set()
    worst = 0.0
    for n, ln in enumerate(lengths):
        ref = oracle_prefix_states(x, n, interval, ln)
        for (nn, toks, slot) in index:
            if nn != n:
                continue
            e = rel(snaps[slot].numpy(), ref[toks // interval - 1])
            worst = max(worst, e)
            assert e <= tol, f"sequence {n}, {toks} tokens, slot {slot}: {e}"
            written.add(slot)
    for s in range(slots):
        if s not in written:
            assert torch.isnan(snaps[s]).all(), f"slot {s} was written but matches no snapshot"
    say(f"snapshots every {interval}: {len(written)} written of {slots} slots, "
        f"worst state rel err {worst:.3e}")
    return xd, out, fin, snaps, index


def test_bf16_snapshots_fixed_length(dev):
    x = small_inputs(torch.bfloat16, 2, 700, 2, 128, 128, 41, init_std=0.02)
    # 64 and 192: per-chunk records; 128 and 512: pair records
    for interval in (64, 128, 192, 512):
        check_case(x, dev, interval, [700, 700], False, 700, TOL_BF16_STATE)


def test_bf16_snapshots_varlen_edges(dev):
    # empty sequence, a length equal to the interval, a multiple of it, ragged ones
    lengths = [300, 0, 128, 512, 70, 1]
    x = small_inputs(torch.bfloat16, 1, 0, 2, 128, 128, 42, lengths=lengths, init_std=0.02)
    check_case(x, dev, 128, lengths, True, None, TOL_BF16_STATE)


def test_bf16_replay_from_snapshot_is_bitwise(dev):
    lengths = [1000]
    x = small_inputs(torch.bfloat16, 1, 1000, 2, 128, 128, 43, init_std=0.02)
    xd, out, fin, snaps, index = check_case(x, dev, 256, lengths, False, 1000, TOL_BF16_STATE)
    snaps = snaps.to(dev)
    for (_, toks, slot) in index:
        rest = {k: xd[k][:, toks:].contiguous() for k in KEYS}
        o2, f2 = kda.chunk_fwd(rest["q"], rest["k"], rest["v"], rest["g"], rest["beta"],
                               rest["z"], init_state=snaps[slot:slot + 1].contiguous())
        torch.cuda.synchronize()
        assert torch.equal(o2, out[:, toks:]), f"replay from {toks} tokens: outputs differ"
        assert torch.equal(f2, fin), f"replay from {toks} tokens: final state differs"
    say(f"replay from {len(index)} snapshots equals the single call bitwise")


def test_f32_snapshots(dev):
    lengths = [64, 37, 0, 96]
    x = small_inputs(torch.float32, 1, 0, 2, 16, 16, 44, lengths=lengths, init_std=0.5)
    check_case(x, dev, 32, lengths, True, None, TOL_F32)
    y = small_inputs(torch.float32, 3, 80, 2, 16, 16, 45)
    check_case(y, dev, 16, [80, 80, 80], False, 80, TOL_F32)
