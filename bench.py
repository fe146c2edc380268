#!/usr/bin/env python3
"""Benchmark of the KDA hot path on one MI355X.

One step = one ``kda_chunk_fwd`` call (prep, chain and output kernels) over the
whole long-context prefill workload: B=1, H=16, T=1,048,576 tokens,
dk=dv=128, bf16 inputs, fp32 state, 64-token chunks, a quarter of the key
channels at the log-decay floor g = -5 (the largest configuration that fits one
GPU).  Inputs are resident in HBM before timing starts; at 4 GiB per tensor
they are far larger than the 256 MB Infinity Cache, so every step reads them
from HBM.

Prints one JSON line:
  value      prefill tokens/s of that workload (T per call / seconds per call)
  roofline   the call against the HBM roof: algorithmic bytes per call
             (1,538 B per token-head + the fp32 final state) / call time, over
             8 TB/s; traffic = HBM bytes per call from rocprofv3 FETCH_SIZE /
             WRITE_SIZE counters, when the committed summary was taken on the
             current kernel sources
  mfma       algorithmic flops per call / call time over the bf16 dense peak
             (and the executed bf16 MFMA flops from counters, when current)
  cpu_baseline  the fp64 oracle on a bounded sample of the same workload, on
             the host cores
Named blocks, timed the same way: prefill_t4096_h8 (B=1, H=8, T=4096),
varlen_4seq_h32 (4 packed sequences, H=32), decode (256 sequences x 32 heads,
512 MiB fp32 state in place, 128 steps), backward_prefill_t4096_h8; extras:
snapshots, the fused prologue, speculative verify / commit.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
                       [--workloads long,prefill,varlen,decode,backward,extras]
       python bench.py --copy-calibration   (a 1 GiB device copy, for counters)
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2516.6
PREFILL_BYTES_PER_TOKEN_HEAD = 1538      # q, k, g, v, z, out at 256 B each + beta at 2 B
STATE_BYTES = 128 * 128 * 4              # one fp32 state slice
DK = DV = 128
CHUNK = 64
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "kda_hbm_traffic.json")
KERNEL_SOURCES = [
    os.path.join(ROOT, "kimi_delta_attention_chunkwise_amd", "csrc", f)
    for f in ("kda_chunk_bf16.hip", "kda_decode.hip", "kda_internal.h", "kda_api.hip",
              "kda_chunk_bwd_bf16.hip")
]
ALL_WORKLOADS = "long,prefill,varlen,decode,backward,extras"


def flops_per_token_head(C=CHUNK, dk=DK, dv=DV):
    """The method's own flops per token-head at chunk C (no masked or padded work):
    6 dk dv (W S, Q~ S, K'^T U) + (3C - 1) dk (A, P, T K) + 2 C dv (T V, P U) + C^2 / 3."""
    return 6 * dk * dv + (3 * C - 1) * dk + 2 * C * dv + C * C / 3.0


# comments, string and character literals of C/C++ source
_C_TOKENS = re.compile(r'//[^\n]*|/\*.*?\*/|"(?:\\.|[^"\\\n])*"|\'(?:\\.|[^\'\\\n])*\'', re.S)


def _code_only(text: str) -> str:
    """The source with comments removed and whitespace runs collapsed, so that
    an edit of a comment does not count as a change of the kernels."""
    text = _C_TOKENS.sub(lambda m: " " if m.group(0)[0] == "/" else m.group(0), text)
    return " ".join(text.split())


def source_digest(paths=KERNEL_SOURCES) -> str:
    h = hashlib.sha256()
    for p in paths:
        with open(p, encoding="utf-8") as fh:
            h.update(_code_only(fh.read()).encode())
    return h.hexdigest()[:16]


def load_traffic(workload, key):
    """A figure of ``workload`` (``hbm_bytes_per_call``, ``hbm_bytes_per_step``,
    ``mfma_executed_bf16_flops_per_call``) from the committed rocprofv3 counter
    summary, if it was taken on the current kernel sources; else None."""
    try:
        with open(TRAFFIC_FILE) as fh:
            t = json.load(fh)
    except (OSError, ValueError):
        return None
    if t.get("source_digest") != source_digest():
        return None
    v = t.get("workloads", {}).get(workload, {}).get(key)
    return None if v is None else float(v)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20,
                    help="timed calls of the headline workload (about 25 ms each)")
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--decode-steps", type=int, default=128)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--workloads", default=ALL_WORKLOADS,
                    help=f"comma-separated subset of {ALL_WORKLOADS} (default: all)")
    return ap.parse_args()


def copy_calibration(torch):
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda")
    src.fill_(1)
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": n, "reps": 5}), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the KDA path here runs on one GPU)",
              file=sys.stderr, flush=True)
        return 2
    import torch

    import kimi_delta_attention_chunkwise_amd as kda
    import workloads as W

    if not torch.cuda.is_available():
        print("bench.py needs a HIP device", file=sys.stderr)
        return 1
    if args.copy_calibration:
        copy_calibration(torch)
        return 0
    dev = torch.device("cuda:0")
    kda.load_library()
    todo = set(args.workloads.split(","))
    result = {
        "metric": "KDA prefill tokens/s + decode steps/s; % bf16 MFMA peak / % HBM GB/s peak",
        "value": None, "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": None, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
    }
    if "long" in todo:
        long = bench_long(torch, kda, W, dev, args)
        result.update(value=long.pop("tokens_per_s"), ms_per_step=long.pop("ms_per_call"))
        result.update(long)
    else:
        result["config"] = {"workload": "long_t1m_h16", "skipped": True}
    if "prefill" in todo:
        result["prefill_t4096_h8"] = bench_prefill(torch, kda, W, dev, args,
                                                   with_extras="extras" in todo)
    if "backward" in todo:
        result["backward_prefill_t4096_h8"] = bench_backward(torch, kda, W, dev, args)
    if "varlen" in todo:
        result["varlen_4seq_h32"] = bench_varlen(torch, kda, W, dev)
    if "decode" in todo:
        result["decode"] = bench_decode(torch, kda, W, dev, args)
        if "extras" in todo:
            result.setdefault("extras", {})["decode_prologue_verify"] = bench_decode_extras(
                torch, kda, W, dev, args)
    result["device"] = device_info(torch, dev)
    if not args.no_cpu_baseline and "long" in todo:
        result["cpu_baseline"] = cpu_baseline(torch, W, dev)
    print(json.dumps(result), flush=True)
    return 0


def prefill_roofline(workload, ms, token_heads, states, kernels):
    """Roofline and MFMA blocks of one forward call: algorithmic bytes (1,538 B per
    token-head + ``states`` fp32 state slices) and flops per call over the event-timed
    call time; HBM traffic and executed MFMA flops from the committed counters when
    they were taken on the current sources."""
    t_s = ms / 1e3
    nbytes = PREFILL_BYTES_PER_TOKEN_HEAD * token_heads + states * STATE_BYTES
    flops = flops_per_token_head() * token_heads
    achieved = nbytes / t_s / 1e9
    roof = {"bound": "hbm", "kernel": kernels, "achieved": achieved, "peak": HBM_PEAK_GBS,
            "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
            "traffic": load_traffic(workload, "hbm_bytes_per_call"),
            "algorithmic_bytes_per_call": nbytes}
    mfma = {"achieved": flops / t_s / 1e12, "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
            "frac": flops / t_s / 1e12 / BF16_PEAK_TFLOPS, "algorithmic_flops_per_call": flops}
    executed = load_traffic(workload, "mfma_executed_bf16_flops_per_call")
    if executed is not None:
        # bf16 MFMA flops the kernels execute (SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512),
        # masked and folded products included, over the same call time
        mfma["executed_flops_per_call"] = executed
        mfma["executed_frac"] = executed / t_s / 1e12 / BF16_PEAK_TFLOPS
    return roof, mfma


def bench_long(torch, kda, W, dev, args):
    """The headline: one kda_chunk_fwd call over the 1M-token workload (B=1,
    H=16, T=2^20, a quarter of the key channels at g = -5, zero initial state,
    final state written), timed over K calls after W warm-up calls."""
    w = W.WORKLOADS["long_t1m_h16"]
    x = W.prefill_inputs(w, device=dev, seed=0)
    B, T, H = w.B, w.T, w.H
    ws = torch.empty(kda.chunk_fwd_workspace_bytes(B, T, B, H, DK, DV, CHUNK, torch.bfloat16,
                                                   False), dtype=torch.uint8, device=dev)
    out = torch.empty(B, T, H, DV, dtype=torch.bfloat16, device=dev)
    fin = torch.empty(B, H, DK, DV, dtype=torch.float32, device=dev)

    def call(i):
        kda.chunk_fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["z"], workspace=ws, out=out,
                      final_state=fin)

    w0 = time.perf_counter()
    ms = _time(torch, call, args.steps, args.warmup)
    wall = time.perf_counter() - w0
    print(f"[bench] long_t1m_h16: {args.steps} calls, {ms:.3f} ms per call "
          f"(wall {wall:.2f} s with {args.warmup} warm-up calls)", file=sys.stderr, flush=True)
    roof, mfma = prefill_roofline("long_t1m_h16", ms, B * T * H, B * H,
                                  "kda_chunk_fwd call (prep + chain + output kernels)")
    res = {"ms_per_call": ms, "tokens_per_s": B * T / (ms / 1e3),
           "config": {"workload": "long_t1m_h16", "B": B, "T": T, "H": H, "dk": DK, "dv": DV,
                      "chunk": CHUNK, "global_batch": B, "seq_len": T, "parallelism": "none",
                      "state": "fp32, zero init, final state written",
                      "pinned_channels": "a quarter of the key channels at g = -5",
                      "workspace_bytes": int(ws.numel())},
           "roofline": roof, "mfma": mfma}
    del x, ws, out, fin
    torch.cuda.empty_cache()
    return res


def bench_prefill(torch, kda, W, dev, args, with_extras=True):
    """prefill_t4096_h8 (B=1, H=8, T=4096): the calls rotate over enough input
    sets (> 600 MiB) that every call reads inputs that are not cache-resident."""
    w = W.WORKLOADS["prefill_t4096_h8"]
    B, T, H = w.B, w.T, w.H
    sets = prefill_sets(W, dev)
    n_sets = len(sets)
    ws = torch.empty(kda.chunk_fwd_workspace_bytes(B, T, B, H, DK, DV, CHUNK, torch.bfloat16,
                                                   False), dtype=torch.uint8, device=dev)
    out = torch.empty(B, T, H, DV, dtype=torch.bfloat16, device=dev)
    fin = torch.empty(B, H, DK, DV, dtype=torch.float32, device=dev)

    def step(i):
        x = sets[i % n_sets]
        kda.chunk_fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["z"], workspace=ws, out=out,
                      final_state=fin)

    steps = max(args.steps, 100)
    ms = _time(torch, step, steps, max(args.warmup, 10))
    print(f"[bench] prefill_t4096_h8: {steps} calls, {ms:.4f} ms per call", file=sys.stderr,
          flush=True)
    roof, mfma = prefill_roofline("prefill_t4096_h8", ms, B * T * H, B * H,
                                  "kda_chunk_fwd call (prep + chain + output kernels)")
    res = {"workload": "prefill_t4096_h8", "B": B, "T": T, "H": H, "input_sets": n_sets,
           "steps": steps, "ms_per_call": ms, "tokens_per_s": B * T / (ms / 1e3),
           "workspace_bytes": int(ws.numel()), "roofline": roof, "mfma": mfma}
    if with_extras:
        res["snapshots_prologue"] = bench_prefill_extras(torch, kda, sets, ws, out, fin, ms, args)
    del sets, ws, out, fin
    return res


def bench_decode(torch, kda, W, dev, args):
    w = W.WORKLOADS["decode_n256_h32"]
    N, H = w.N, w.H
    state = W.decode_init_state(w, device=dev)
    n_sets = 8
    sets = [W.decode_inputs(w, step=s, device=dev) for s in range(n_sets)]
    out = torch.empty(N, H, DV, dtype=torch.bfloat16, device=dev)

    def step(i):
        x = sets[i % n_sets]
        kda.decode_step(x["q"], x["k"], x["v"], x["g"], x["beta"], x["z"], state, out=out)

    for i in range(max(4, args.warmup // 4)):
        step(i)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(args.decode_steps):
        step(i)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.decode_steps
    print(f"[bench] decode timed: {args.decode_steps} steps, {ms:.4f} ms/step",
          file=sys.stderr, flush=True)
    bytes_step = N * H * (2 * STATE_BYTES + PREFILL_BYTES_PER_TOKEN_HEAD)
    gbs = bytes_step / (ms / 1e3) / 1e9
    measured = measured_bandwidth(torch, state)
    return {"workload": "decode_n256_h32", "N": N, "H": H, "steps": args.decode_steps,
            "ms_per_step": ms, "steps_per_s": 1e3 / ms, "tokens_per_s": N * 1e3 / ms,
            "roofline": {"bound": "hbm", "kernel": "kda_decode_kernel", "achieved": gbs,
                         "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": gbs / HBM_PEAK_GBS,
                         "traffic": load_traffic("decode_n256_h32", "hbm_bytes_per_step"),
                         "algorithmic_bytes_per_step": bytes_step},
            "measured_bandwidth": dict(measured, decode_frac_of_inplace=gbs / measured["inplace_gbs"])}


def measured_bandwidth(torch, state):
    """Secondary denominators measured on this device with torch's own kernels:
    a 1 GiB device-to-device copy, and an in-place multiply over a buffer the
    size of the decode state (512 MiB fp32, read and written like the state).
    Read plus write bytes per second."""
    def rate(fn, nbytes, reps=10):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return nbytes / (e0.elapsed_time(e1) / reps / 1e3) / 1e9

    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device=state.device)
    src.fill_(1)
    dst = torch.empty_like(src)
    copy_gbs = rate(lambda: dst.copy_(src), 2 * n)
    del src, dst
    buf = torch.ones_like(state)
    inplace_gbs = rate(lambda: buf.mul_(0.999), 2 * buf.numel() * 4)
    del buf
    return {"copy_1GiB_gbs": copy_gbs, "inplace_gbs": inplace_gbs,
            "inplace_bytes": int(state.numel() * 4)}


def _time(torch, fn, steps, warmup):
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(steps):
        fn(warmup + i)
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def bench_prefill_extras(torch, kda, sets, ws, out, fin, ms_plain, args):
    """The same prefill call with fp32 state snapshots every 512 tokens, and
    with the fused prologue on raw inputs (all three maps)."""
    n_sets = len(sets)
    x0 = sets[0]
    B, T, H, dk = x0["q"].shape
    snaps = torch.empty(kda.snapshot_slots(B, T, B, CHUNK, 512, False), H, dk, DV,
                        dtype=torch.float32, device=x0["q"].device)

    def snap(i):
        x = sets[i % n_sets]
        kda.chunk_fwd_snapshots(x["q"], x["k"], x["v"], x["g"], x["beta"], x["z"], 512,
                                workspace=ws, out=out, final_state=fin, snapshots=snaps)

    ms_snap = _time(torch, snap, max(20, args.steps // 4), 5)
    # raw projections: unnormalised q/k, beta logits, g pre-activations
    gen = torch.Generator(device=x0["q"].device).manual_seed(7)
    raw = [{key: torch.randn(x0[key].shape, generator=gen, device=x0["q"].device).to(
        torch.bfloat16) for key in ("q", "k", "g", "beta")} for _ in range(4)]

    def pro(i):
        x, r = sets[i % n_sets], raw[i % 4]
        kda.chunk_fwd(r["q"], r["k"], x["v"], r["g"], r["beta"], x["z"], workspace=ws, out=out,
                      final_state=fin, prologue=7)

    ms_pro = _time(torch, pro, max(20, args.steps // 4), 5)
    print(f"[bench] prefill with snapshots every 512: {ms_snap:.4f} ms; with prologue: "
          f"{ms_pro:.4f} ms", file=sys.stderr, flush=True)
    return {"workload": "prefill_t4096_h8", "plain_ms": ms_plain,
            "snapshots_every_512_ms": ms_snap,
            "snapshot_bytes_per_call": int(snaps.numel() * 4),
            "prologue_all_ms": ms_pro,
            "prologue_tokens_per_s": B * T / (ms_pro / 1e3)}


def prefill_sets(W, dev):
    """Input sets of prefill_t4096_h8, enough of them (> 600 MiB in all) that
    calls rotating over them read inputs that are not cache-resident."""
    w = W.WORKLOADS["prefill_t4096_h8"]
    in_bytes_per_set = w.B * w.T * w.H * (5 * 256 + 2)
    n_sets = max(2, -(-600 * 2 ** 20 // in_bytes_per_set))      # > 2x the 256 MB MALL
    return [W.prefill_inputs(w, device=dev, seed=s) for s in range(n_sets)]


def bench_backward(torch, kda, W, dev, args):
    """kda_chunk_bwd on the prefill workload: gradients of every input and of
    the initial state from dY ~ N(0, 1) and a zero dS_final, all buffers
    preallocated, rotating over the prefill input sets."""
    sets = prefill_sets(W, dev)
    x0 = sets[0]
    B, T, H, _ = x0["q"].shape
    dev = x0["q"].device
    gen = torch.Generator(device=dev).manual_seed(77)
    dys = [torch.randn(x0["v"].shape, generator=gen, device=dev).to(torch.bfloat16)
           for _ in range(2)]
    ws = torch.empty(kda.chunk_bwd_workspace_bytes(B, T, B, H, DK, DV, CHUNK, torch.bfloat16,
                                                   False), dtype=torch.uint8, device=dev)
    grads = {n: torch.empty_like(x0[src]) for n, src in
             (("q", "q"), ("k", "k"), ("v", "v"), ("g", "g"), ("beta", "beta"), ("gate", "z"))}
    grads["init_state"] = torch.empty(B, H, DK, DV, dtype=torch.float32, device=dev)
    n_sets = len(sets)

    def call(i):
        x = sets[i % n_sets]
        kda.chunk_bwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["z"], dys[i % 2],
                      workspace=ws, grads=grads)

    steps = max(5, args.steps // 2)
    ms = _time(torch, call, steps, max(3, args.warmup // 2))
    print(f"[bench] backward prefill_t4096_h8: {ms:.4f} ms per call", file=sys.stderr,
          flush=True)
    # a training step: the forward, then the backward reusing the forward's records
    ws_fwd = torch.empty(kda.chunk_fwd_workspace_bytes(B, T, B, H, DK, DV, CHUNK,
                                                       torch.bfloat16, False, chunk_records=True),
                         dtype=torch.uint8, device=dev)
    ws_half = torch.empty(ws.numel() - ws_fwd.numel(), dtype=torch.uint8, device=dev)
    out = torch.empty_like(x0["v"])

    def train_step(i):
        # the forward keeps per-chunk records, which the backward then reuses
        x = sets[i % n_sets]
        kda.chunk_fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["z"], workspace=ws_fwd,
                      out=out, output_final_state=False, chunk_records=True)
        kda.chunk_bwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["z"], dys[i % 2],
                      workspace=ws_half, grads=grads, fwd_workspace=ws_fwd)

    ms_train = _time(torch, train_step, steps, max(3, args.warmup // 2))

    def fwd(i):
        x = sets[i % n_sets]
        kda.chunk_fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["z"], workspace=ws_fwd,
                      out=out, output_final_state=False)

    ms_fwd = _time(torch, fwd, max(20, steps), 5)
    print(f"[bench] forward + backward on the forward's records: {ms_train:.4f} ms",
          file=sys.stderr, flush=True)
    token_heads = B * T * H
    # reads q, k, v, g, z, dY (256 B each) and beta; writes dq, dk, dv, dg, dz and dbeta;
    # the fp32 dS_0
    bytes_call = (6 * 256 + 2 + 5 * 256 + 2) * token_heads + B * H * STATE_BYTES
    flops_call = 3 * flops_per_token_head() * token_heads
    t_s = ms / 1e3
    del ws, grads, ws_fwd, ws_half, sets
    return {"workload": "prefill_t4096_h8", "ms_per_call": ms, "tokens_per_s": B * T / t_s,
            "forward_ms": ms_fwd, "ratio_to_forward": ms / ms_fwd, "steps": steps,
            "train_step_ms": ms_train, "train_step_tokens_per_s": B * T / (ms_train / 1e3),
            "train_step": "kda_chunk_fwd_ex with per-chunk records, then kda_chunk_bwd_ex "
                          "on them",
            "kernels": "forward prep + chain, backward prep, chain, gradient kernel",
            "roofline": {"bound": "hbm", "achieved": bytes_call / t_s / 1e9,
                         "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": bytes_call / t_s / 1e9 / HBM_PEAK_GBS,
                         "traffic": load_traffic("backward_prefill_t4096_h8",
                                                 "hbm_bytes_per_call"),
                         "algorithmic_bytes_per_call": bytes_call},
            "mfma": {"achieved": flops_call / t_s / 1e12, "peak": BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": flops_call / t_s / 1e12 / BF16_PEAK_TFLOPS,
                     "executed_flops_per_call": load_traffic("backward_prefill_t4096_h8",
                                                             "mfma_executed_bf16_flops_per_call"),
                     "algorithmic_flops_per_call": flops_call,
                     "flops_rule": "3 x the forward's: the recompute plus two products of "
                                   "the same size for the adjoint of each product"}}


def bench_decode_extras(torch, kda, W, dev, args):
    """Decode step with the fused prologue, and speculative verification of
    K = 4 draft tokens followed by a commit of all of them, on the decode
    workload's 512 MiB state."""
    w = W.WORKLOADS["decode_n256_h32"]
    N, H, K = w.N, w.H, 4
    state = W.decode_init_state(w, device=dev)
    gen = torch.Generator(device=dev).manual_seed(11)
    r = lambda *s: torch.randn(*s, generator=gen, device=dev).to(torch.bfloat16)
    one = {"q": r(N, H, DK), "k": r(N, H, DK), "v": r(N, H, DV), "g": r(N, H, DK),
           "beta": r(N, H), "z": r(N, H, DV)}
    out = torch.empty(N, H, DV, dtype=torch.bfloat16, device=dev)

    def step(i):
        kda.decode_step(one["q"], one["k"], one["v"], one["g"], one["beta"], one["z"], state,
                        out=out, prologue=7)

    ms_pro = _time(torch, step, 32, 4)
    x = W.decode_inputs(w, step=0, device=dev)
    drafts = {key: torch.stack([x[key]] * K, dim=1).contiguous() for key in x}
    vout = torch.empty(N, K, H, DV, dtype=torch.bfloat16, device=dev)
    u = torch.empty(N, K, H, DV, dtype=torch.float32, device=dev)
    acc = torch.full((N,), K, dtype=torch.int32, device=dev)

    def verify(i):
        kda.decode_verify(drafts["q"], drafts["k"], drafts["v"], drafts["g"], drafts["beta"],
                          drafts["z"], state, out=vout, u=u)

    def commit(i):
        kda.decode_commit(drafts["k"], drafts["g"], u, acc, state)

    ms_ver = _time(torch, verify, 32, 4)
    ms_com = _time(torch, commit, 32, 4)
    print(f"[bench] decode with prologue: {ms_pro:.4f} ms; verify K={K}: {ms_ver:.4f} ms; "
          f"commit: {ms_com:.4f} ms", file=sys.stderr, flush=True)
    return {"workload": "decode_n256_h32", "prologue_all_step_ms": ms_pro,
            "verify_draft_tokens": K, "verify_ms": ms_ver, "commit_all_ms": ms_com,
            "verified_tokens_per_s": N * K / ((ms_ver + ms_com) / 1e3)}


def bench_varlen(torch, kda, W, dev, calls=10):
    """The packed varlen workload: 4 sequences (lengths drawn uniform in
    [1024, 32768], seed 0) in one cu_seqlens call, H=32, fp32 initial state
    N(0, 0.02^2), final state written."""
    w = W.WORKLOADS["varlen_4seq_h32"]
    x = W.prefill_inputs(w, device=dev, seed=0)
    lens = W.varlen_lengths(w, 0)
    T, H, N = int(sum(lens)), w.H, len(lens)
    ws = torch.empty(kda.chunk_fwd_workspace_bytes(1, T, N, H, DK, DV, CHUNK, torch.bfloat16,
                                                   True), dtype=torch.uint8, device=dev)
    out = torch.empty(1, T, H, DV, dtype=torch.bfloat16, device=dev)
    fin = torch.empty(N, H, DK, DV, dtype=torch.float32, device=dev)

    def call(i):
        kda.chunk_fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["z"],
                      init_state=x["init_state"], cu_seqlens=x["cu_seqlens"], workspace=ws,
                      out=out, final_state=fin)

    ms = _time(torch, call, calls, 2)
    print(f"[bench] varlen_4seq_h32 (lengths {lens}): {ms:.3f} ms per call", file=sys.stderr,
          flush=True)
    # state I/O: the fp32 initial state is read and the final state written
    roof, mfma = prefill_roofline("varlen_4seq_h32", ms, T * H, 2 * N * H,
                                  "kda_chunk_fwd call (prep + chain + output kernels)")
    nbytes = int(ws.numel())
    del x, ws, out
    return {"workload": "varlen_4seq_h32", "lengths": lens, "calls": calls, "ms_per_call": ms,
            "tokens_per_s": T / (ms / 1e3), "workspace_bytes": nbytes, "roofline": roof,
            "mfma": mfma}


def device_info(torch, dev):
    """The device the numbers were taken on: name, architecture, compute units,
    peak shader clock (HIP's hipDeviceAttributeClockRate, enum value 5, kHz)
    and memory, against which the peaks above are quoted."""
    p = torch.cuda.get_device_properties(dev)
    info = {"name": p.name, "arch": p.gcnArchName, "compute_units": p.multi_processor_count,
            "memory_gib": round(p.total_memory / 2 ** 30, 1), "peak_clock_mhz": None}
    try:
        import ctypes
        # by soname: the HIP runtime torch has already loaded, not a second copy
        hip = ctypes.CDLL("libamdhip64.so.7")
        khz = ctypes.c_int(0)
        if hip.hipDeviceGetAttribute(ctypes.byref(khz), 5, dev.index or 0) == 0:
            info["peak_clock_mhz"] = khz.value / 1000.0
    except OSError:
        pass
    return info


def cpu_baseline(torch, W, dev):
    """The fp64 oracle (as it stands) on a bounded sample of the headline
    workload: the first tokens of long_t1m_h16, all 16 heads, in consecutive
    segments of 32,768 tokens (the same inputs the GPU ran, widened exactly
    from bf16 to float32 on the host), the state carried from segment to
    segment, until about 10 s have passed; OpenMP over the 16 heads.  Also the
    one-thread rate on one head, and the oracle's decode rate."""
    import numpy as np

    import oracle
    w = W.WORKLOADS["long_t1m_h16"]
    x = W.prefill_inputs(w, device=dev, seed=0)
    keys = ("q", "k", "v", "g", "beta", "z")
    threads = max(1, min(os.cpu_count() or 1, 16))
    seg = 32768
    state = None
    tokens, elapsed = 0, 0.0
    while elapsed < 10.0 and tokens + seg <= w.T:
        arrs = [x[k][:, tokens:tokens + seg].float().cpu().numpy() for k in keys]
        t0 = time.perf_counter()
        _, state = oracle.forward(*arrs, init_state=state, n_threads=threads)
        elapsed += time.perf_counter() - t0
        tokens += seg
    # one thread, one head, about 3 s
    one = [x[k][:, :seg, :1].float().cpu().numpy() for k in keys]
    t1, e1 = 0, 0.0
    while e1 < 3.0 and t1 < 64:
        t0 = time.perf_counter()
        oracle.forward(*one, n_threads=1)
        e1 += time.perf_counter() - t0
        t1 += 1
    del x, one
    torch.cuda.empty_cache()
    # decode_n256_h32 (256 sequences x 32 heads, fp64 state in place): a few steps
    wd = W.WORKLOADS["decode_n256_h32"]
    st = W.decode_init_state(wd, device="cpu", seed=0).double().numpy()
    dins = []
    for i in range(8):
        xd = W.decode_inputs(wd, i, device="cpu", seed=0)
        dins.append([xd[k].float().numpy() for k in keys])
    dsteps, delapsed = 0, 0.0
    while delapsed < 4.0 and dsteps < 4096:
        t0 = time.perf_counter()
        oracle.decode_step(*dins[dsteps % 8], st, n_threads=threads)
        delapsed += time.perf_counter() - t0
        dsteps += 1
    del st, dins
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), "")
    except OSError:
        pass
    del np
    return {"value": tokens / elapsed, "unit": "tokens/s", "cores": min(threads, w.H),
            "kind": "oracle",
            "sample": f"long_t1m_h16: the first {tokens:,} of its {w.T:,} tokens, all {w.H} heads, "
                      f"in segments of {seg:,} tokens with the state carried, {elapsed:.1f} s; "
                      f"OpenMP over the {w.H} heads with {min(threads, w.H)} threads",
            "single_thread_value": t1 * seg / e1,
            "single_thread_sample": f"one head, {seg:,} tokens, {t1} calls, one thread; "
                                    "tokens/s of that head alone",
            "decode_steps_per_s": dsteps / delapsed,
            "decode_sample": f"decode_n256_h32, {dsteps} steps (8 input sets in turn) of the "
                             f"fp64 oracle on the full state, {delapsed:.1f} s, OpenMP over the "
                             f"{wd.N * wd.H} (sequence, head) units with {threads} threads",
            "host_cpus": os.cpu_count(), "cpu_model": model}


if __name__ == "__main__":
    sys.exit(main())
