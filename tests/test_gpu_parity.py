"""GPU parity: the HIP path through the C ABI against the fp64 CPU oracle.

Both sides get the very same tensors (drawn once by ``workloads``; the oracle
sees them widened exactly to float32).  The error measure is
max|x - ref| / max|ref| over a whole tensor.  Tolerances: 2e-2 on outputs and
1e-2 on final states for bf16 inputs with an fp32 state, 1e-4 on both for the
fp32 path.
"""
from __future__ import annotations

import os

import numpy as np
import pytest
import torch

import kimi_delta_attention_chunkwise_amd as kda
import oracle
import workloads as W

pytestmark = pytest.mark.gpu

TOL_BF16_OUT, TOL_BF16_STATE = 2e-2, 1e-2
TOL_F32 = 1e-4


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no HIP device")
    kda.load_library()            # raises if libkda.so is missing: no silent fallback
    return torch.device("cuda:0")


def say(msg):
    print(f"[gpu-parity] {msg}", flush=True)


def np32(t):
    return None if t is None else t.detach().to("cpu", torch.float32).numpy()


def rel(x, ref):
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = float(np.max(np.abs(ref))) if ref.size else 0.0
    if ref.size == 0:
        return 0.0
    return float(np.max(np.abs(x - ref)) / (den if den > 0 else 1.0))


def to(d, dev):
    return {k: (v.to(dev) if isinstance(v, torch.Tensor) else v) for k, v in d.items()}


def run_gpu(x, dev, **kw):
    x = to(x, dev)
    out, fin = kda.chunk_fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["z"],
                             init_state=x.get("init_state"), cu_seqlens=x.get("cu_seqlens"), **kw)
    torch.cuda.synchronize()
    return out, fin


def run_oracle(x, scale=1.0, threads=None):
    cu = x.get("cu_seqlens")
    return oracle.forward(np32(x["q"]), np32(x["k"]), np32(x["v"]), np32(x["g"]), np32(x["beta"]),
                          np32(x["z"]), init_state=np32(x.get("init_state")),
                          cu_seqlens=None if cu is None else cu.cpu().numpy(), scale=scale,
                          n_threads=threads)


def check(out, fin, ref_out, ref_fin, tol_out, tol_state, label):
    eo = rel(np32(out), ref_out)
    es = rel(np32(fin), ref_fin) if fin is not None else 0.0
    say(f"{label}: out rel err {eo:.3e}, state rel err {es:.3e}")
    assert np.all(np.isfinite(np32(out)))
    assert eo <= tol_out, f"{label}: output error {eo}"
    assert es <= tol_state, f"{label}: state error {es}"


def worst_slice(x, ref, kind, cu=None):
    """The (sequence, head) slice with the largest max|x - ref| / max|ref|.
    kind "out": x, ref are [B, T, H, d] outputs, sliced per (batch row, head),
    or per (sequence of cu, head) when cu is given; kind "state": [N, H, dk, dv]
    states, sliced per (n, h).  Returns (error, (n, h))."""
    x, ref = np.asarray(x, dtype=np.float64), np.asarray(ref, dtype=np.float64)
    if kind == "state":
        slices = [((n, h), x[n, h], ref[n, h]) for n in range(x.shape[0])
                  for h in range(x.shape[1])]
    elif cu is not None:
        cu = np.asarray(cu)
        slices = [((n, h), x[0, cu[n]:cu[n + 1], h], ref[0, cu[n]:cu[n + 1], h])
                  for n in range(len(cu) - 1) for h in range(x.shape[2])]
    else:
        slices = [((n, h), x[n, :, h], ref[n, :, h]) for n in range(x.shape[0])
                  for h in range(x.shape[2])]
    best = (0.0, (0, 0))
    for nh, xs, rs in slices:
        if rs.size:
            err = rel(xs, rs)
            if err > best[0]:
                best = (err, nh)
    return best


def log_worst(label, out, ref_out, fin=None, ref_fin=None, cu=None):
    eo, nho = worst_slice(np32(out), ref_out, "out", cu)
    msg = f"{label}: worst (n, h) out slice {nho} rel err {eo:.3e}"
    if fin is not None:
        es, nhs = worst_slice(np32(fin), ref_fin, "state")
        msg += f"; worst state slice {nhs} rel err {es:.3e}"
    say(msg)


def small_inputs(dtype, B, T, H, dk, dv, seed, lengths=None, init_std=0.0, g_mode="random"):
    """Inputs with the workload distributions at custom sizes."""
    gen = torch.Generator().manual_seed(seed)
    if lengths is not None:
        tok = (1, int(sum(lengths)))
        cu = torch.tensor(np.concatenate([[0], np.cumsum(lengths)]), dtype=torch.int32)
        N = len(lengths)
    else:
        tok, cu, N = (B, T), None, B
    pinned = None
    if g_mode == "pinned":
        pinned = torch.zeros(H, dk, dtype=torch.bool)
        for h in range(H):
            pinned[h, torch.randperm(dk, generator=gen)[: dk // 4]] = True
    d = W.draw_tokens(tok, H, dk, dv, dtype, gen, "cpu", pinned)
    if g_mode == "zero":
        d["g"] = torch.zeros_like(d["g"])
    elif g_mode == "slow":
        d["g"] = (d["g"].float() * 0.01).to(dtype)
    elif g_mode == "pinned":
        d["g"] = torch.where(pinned, d["g"].float(), torch.zeros_like(d["g"].float())).to(dtype)
    d["cu_seqlens"] = cu
    d["init_state"] = (torch.randn(N, H, dk, dv, generator=gen) * init_std) if init_std else None
    return d


# ------------------------------------------------------------------ fp32 path
def test_tiny_f32_workload(dev):
    w = W.WORKLOADS["tiny_f32"]
    say("tiny_f32 B=1 H=2 T=64 dk=dv=16 chunk=16")
    x = W.prefill_inputs(w, seed=0)
    out, fin = run_gpu(x, dev, chunk=16)
    ro, rf = run_oracle(x)
    check(out, fin, ro, rf, TOL_F32, TOL_F32, "tiny_f32")


@pytest.mark.parametrize("case", ["varlen_init", "ragged_batch", "zero_decay"])
def test_f32_edge_cases(dev, case):
    say(f"f32 edge case {case}")
    if case == "varlen_init":
        x = small_inputs(torch.float32, 1, 0, 3, 16, 16, 1, lengths=[0, 5, 16, 37, 1],
                         init_std=0.5)
    elif case == "ragged_batch":
        x = small_inputs(torch.float32, 3, 45, 2, 16, 16, 2, init_std=0.3)
    else:
        x = small_inputs(torch.float32, 1, 80, 2, 16, 16, 3, init_std=0.3, g_mode="zero")
    out, fin = run_gpu(x, dev, chunk=16, scale=0.75)
    ro, rf = run_oracle(x, scale=0.75)
    check(out, fin, ro, rf, TOL_F32, TOL_F32, f"f32 {case}")


# ------------------------------------------------------------------ bf16 path
@pytest.mark.parametrize("case", ["ragged_batch", "varlen_edges", "slow_decay", "no_decay",
                                  "pinned_floor"])
def test_bf16_small_cases(dev, case):
    say(f"bf16 case {case}")
    bf = torch.bfloat16
    if case == "ragged_batch":
        x = small_inputs(bf, 2, 200, 2, 128, 128, 10, init_std=0.02)
    elif case == "varlen_edges":
        x = small_inputs(bf, 1, 0, 3, 128, 128, 11, lengths=[0, 1, 63, 64, 65, 129, 300, 0],
                         init_std=0.02)
    elif case == "slow_decay":
        x = small_inputs(bf, 1, 640, 2, 128, 128, 12, init_std=0.02, g_mode="slow")
    elif case == "no_decay":
        x = small_inputs(bf, 1, 320, 2, 128, 128, 13, init_std=0.02, g_mode="zero")
    else:
        x = small_inputs(bf, 1, 256, 2, 128, 128, 14, init_std=0.02, g_mode="pinned")
    out, fin = run_gpu(x, dev)
    ro, rf = run_oracle(x)
    check(out, fin, ro, rf, TOL_BF16_OUT, TOL_BF16_STATE, f"bf16 {case}")


@pytest.mark.parametrize("g_mode", ["slow", "zero"])
def test_bf16_long_slow_decay(dev, g_mode):
    """16,384 tokens with little or no decay, so every chunk's entry state
    matters to its outputs: 128 steps of the serial pass over composed pairs
    of chunks (and a ragged second sequence), against the oracle."""
    say(f"bf16 long sequences with g_mode={g_mode}: B=2 T=16,333 H=2")
    x = small_inputs(torch.bfloat16, 2, 16_333, 2, 128, 128, 24, init_std=0.02, g_mode=g_mode)
    out, fin = run_gpu(x, dev)
    ro, rf = run_oracle(x)
    check(out, fin, ro, rf, TOL_BF16_OUT, TOL_BF16_STATE, f"bf16 long {g_mode} decay")
    log_worst(f"bf16 long {g_mode} decay", out, ro, fin, rf)


def test_bf16_scale_inplace_state_and_no_final(dev):
    say("bf16 scale 0.5, final_state aliasing init_state, then no final state")
    x = small_inputs(torch.bfloat16, 1, 130, 2, 128, 128, 15, init_std=0.02)
    ro, rf = run_oracle(x, scale=0.5)
    xd = to(x, dev)
    st = xd["init_state"].clone()
    out, fin = kda.chunk_fwd(xd["q"], xd["k"], xd["v"], xd["g"], xd["beta"], xd["z"],
                             init_state=st, final_state=st, scale=0.5)
    torch.cuda.synchronize()
    assert fin.data_ptr() == st.data_ptr()
    check(out, fin, ro, rf, TOL_BF16_OUT, TOL_BF16_STATE, "bf16 in-place state")
    out2, fin2 = kda.chunk_fwd(xd["q"], xd["k"], xd["v"], xd["g"], xd["beta"], xd["z"],
                               init_state=xd["init_state"], output_final_state=False, scale=0.5)
    torch.cuda.synchronize()
    assert fin2 is None
    assert torch.equal(out2, out)


def test_empty_sequences(dev):
    say("empty inputs: T = 0 and all-zero-length varlen")
    x = small_inputs(torch.bfloat16, 1, 0, 2, 128, 128, 16, lengths=[0, 0, 0], init_std=0.1)
    out, fin = run_gpu(x, dev)
    assert out.shape == (1, 0, 2, 128)
    assert torch.equal(fin.cpu(), x["init_state"])
    x = small_inputs(torch.bfloat16, 2, 0, 2, 128, 128, 17)
    out, fin = run_gpu(x, dev)
    assert torch.count_nonzero(fin) == 0


def test_misaligned_input_is_refused(dev):
    """A contiguous q that starts one element into its buffer is below the
    16-byte alignment: the call is refused on the host and writes nothing."""
    say("misaligned q: refused before launch")
    x = to(small_inputs(torch.bfloat16, 1, 64, 2, 128, 128, 18), dev)
    flat = torch.empty(x["q"].numel() + 8, dtype=torch.bfloat16, device=dev)
    q = flat[1:1 + x["q"].numel()].view(x["q"].shape)
    q.copy_(x["q"])
    out = torch.full_like(x["v"], 7.0)
    with pytest.raises(kda.KdaError, match="KDA_ERR_MISALIGNED"):
        kda.chunk_fwd(q, x["k"], x["v"], x["g"], x["beta"], x["z"], out=out)
    torch.cuda.synchronize()
    assert torch.all(out == 7.0)


def test_bf16_split_equals_single_call(dev):
    say("bf16 split at T/2 (aligned) and at an unaligned point")
    x = small_inputs(torch.bfloat16, 1, 512, 2, 128, 128, 18, init_std=0.02)
    xd = to(x, dev)
    full_out, full_fin = kda.chunk_fwd(xd["q"], xd["k"], xd["v"], xd["g"], xd["beta"], xd["z"],
                                       init_state=xd["init_state"])
    for tau in (256, 200):
        keys = ("q", "k", "v", "g", "beta", "z")
        a = {k: xd[k][:, :tau].contiguous() for k in keys}
        b = {k: xd[k][:, tau:].contiguous() for k in keys}
        o1, s1 = kda.chunk_fwd(a["q"], a["k"], a["v"], a["g"], a["beta"], a["z"],
                               init_state=xd["init_state"])
        o2, s2 = kda.chunk_fwd(b["q"], b["k"], b["v"], b["g"], b["beta"], b["z"], init_state=s1)
        torch.cuda.synchronize()
        cat = torch.cat([o1, o2], dim=1)
        if tau % 64 == 0:
            # chunk boundaries coincide: identical arithmetic, bitwise equal
            assert torch.equal(cat, full_out) and torch.equal(s2, full_fin)
        else:
            assert rel(np32(cat), np32(full_out)) < 1e-2
            assert rel(np32(s2), np32(full_fin)) < 1e-2


def test_bf16_deterministic(dev):
    say("bf16 run-to-run determinism")
    x = small_inputs(torch.bfloat16, 1, 1000, 4, 128, 128, 19, init_std=0.02)
    o1, f1 = run_gpu(x, dev)
    o2, f2 = run_gpu(x, dev)
    assert torch.equal(o1, o2) and torch.equal(f1, f2)


# ---------------------------------------------------------------- decode
@pytest.mark.parametrize("dtype,d,tol", [(torch.float32, 16, 1e-5), (torch.float32, 128, 1e-5),
                                         (torch.bfloat16, 16, 1e-4), (torch.bfloat16, 128, 1e-4)])
def test_decode_steps_small(dev, dtype, d, tol):
    say(f"decode {dtype} d={d} N=5 H=3, 20 steps, random init")
    gen = torch.Generator().manual_seed(20 + d)
    N, H, steps = 5, 3, 20
    st64 = np.ascontiguousarray(np.random.default_rng(d).standard_normal((N, H, d, d)) * 0.05)
    st = torch.tensor(st64, dtype=torch.float32, device=dev)
    st64 = np32(st).astype(np.float64)            # the oracle starts from the same fp32 state
    for s in range(steps):
        x = W.draw_tokens((N,), H, d, d, dtype, gen, "cpu")
        xd = to(x, dev)
        y = kda.decode_step(xd["q"], xd["k"], xd["v"], xd["g"], xd["beta"], xd["z"], st,
                            scale=0.9)
        ry = oracle.decode_step(np32(x["q"]), np32(x["k"]), np32(x["v"]), np32(x["g"]),
                                np32(x["beta"]), np32(x["z"]), st64, scale=0.9)
        torch.cuda.synchronize()
        # bf16 outputs carry their own rounding (2^-9 relative)
        out_tol = tol if dtype == torch.float32 else 8e-3
        assert rel(np32(y), ry) <= out_tol, s
    es = rel(np32(st), st64)
    say(f"decode state rel err {es:.3e}")
    assert es <= tol


@pytest.mark.parametrize("dtype,d,tol", [(torch.float32, 16, 1e-5), (torch.bfloat16, 128, 1e-4)])
def test_decode_neg_inf_and_zero_log_decay(dev, dtype, d, tol):
    """The decode step has no lower bound on g: a log-decay of -inf gives a
    decay of 0.  Step 1 puts -inf on a quarter of the key channels of every
    (sequence, head); step 3 puts it on every channel of some (sequence,
    head) pairs, which resets their state to the token's own write; step 4
    gives g = 0 (no decay) to others.  Every step is checked against the
    oracle, and the reset pairs also against k (beta v)^T directly."""
    say(f"decode {dtype} d={d}: g = -inf on channels and whole tokens, g = 0")
    gen = torch.Generator().manual_seed(30 + d)
    N, H, steps = 6, 3, 6
    st = (torch.randn(N, H, d, d, generator=gen) * 0.05).to(dev)
    st64 = np32(st).astype(np.float64)
    chan = torch.randperm(d, generator=gen)[: d // 4]
    reset = [(0, 0), (2, 1), (5, 2)]
    for s in range(steps):
        x = W.draw_tokens((N,), H, d, d, dtype, gen, "cpu")
        g = x["g"].float()
        if s == 1:
            g[:, :, chan] = -float("inf")
        if s == 3:
            for n, h in reset:
                g[n, h] = -float("inf")
        if s == 4:
            g[1:4] = 0.0
        x["g"] = g.to(dtype)
        xd = to(x, dev)
        y = kda.decode_step(xd["q"], xd["k"], xd["v"], xd["g"], xd["beta"], xd["z"], st,
                            scale=0.9)
        ry = oracle.decode_step(np32(x["q"]), np32(x["k"]), np32(x["v"]), np32(x["g"]),
                                np32(x["beta"]), np32(x["z"]), st64, scale=0.9)
        torch.cuda.synchronize()
        ey, es = rel(np32(y), ry), rel(np32(st), st64)
        say(f"  step {s}: out rel err {ey:.3e}, state rel err {es:.3e}")
        assert np.all(np.isfinite(np32(y))) and np.all(np.isfinite(np32(st)))
        assert ey <= (tol if dtype == torch.float32 else 8e-3) and es <= tol, s
        if s == 3:
            k64, v64, b64 = (np32(x[key]).astype(np.float64) for key in ("k", "v", "beta"))
            stn = np32(st)
            for n, h in reset:
                want = np.outer(k64[n, h], b64[n, h] * v64[n, h])
                assert rel(stn[n, h], want) <= tol, (n, h)


@pytest.mark.parametrize("dtype,d,tol", [(torch.float32, 16, 1e-5), (torch.bfloat16, 128, 1e-4)])
def test_decode_prologue_infinite_decay_inputs(dev, dtype, d, tol):
    """With the softplus prologue, a pre-activation of +inf maps to the floor
    g = -5 and -inf maps to g = 0 (decay 1); q and k are normalised and beta is
    a logit.  Checked against the prologue oracle followed by the recurrence."""
    from oracle import prologue as P
    say(f"decode prologue {dtype} d={d}: g pre-activations of +inf and -inf")
    gen = torch.Generator().manual_seed(40 + d)
    N, H, steps = 4, 3, 4
    st = (torch.randn(N, H, d, d, generator=gen) * 0.05).to(dev)
    st64 = np32(st).astype(np.float64)
    for s in range(steps):
        raw = {key: (torch.randn(N, H, d if key != "beta" else 1, generator=gen) * 2).squeeze(-1)
               for key in ("q", "k", "g", "beta")}
        raw["g"][:, :, : d // 4] = float("inf")
        raw["g"][:, :, d // 4: d // 2] = -float("inf")
        raw["v"] = torch.randn(N, H, d, generator=gen)
        raw["z"] = torch.randn(N, H, d, generator=gen)
        x = {key: val.to(dtype) for key, val in raw.items()}
        xd = to(x, dev)
        y = kda.decode_step(xd["q"], xd["k"], xd["v"], xd["g"], xd["beta"], xd["z"], st,
                            prologue=kda.PRO_QK_L2NORM | kda.PRO_BETA_SIGMOID |
                            kda.PRO_G_SOFTPLUS)
        q, k, beta, g = P.apply(np32(x["q"]), np32(x["k"]), np32(x["beta"]), np32(x["g"]), 7)
        assert np.all(g[:, :, : d // 4] == -5.0) and np.all(g[:, :, d // 4: d // 2] == 0.0)
        ry = oracle.decode_step(q, k, np32(x["v"]).astype(np.float64), g, beta,
                                np32(x["z"]).astype(np.float64), st64)
        torch.cuda.synchronize()
        ey, es = rel(np32(y), ry), rel(np32(st), st64)
        say(f"  step {s}: out rel err {ey:.3e}, state rel err {es:.3e}")
        assert np.all(np.isfinite(np32(y))) and np.all(np.isfinite(np32(st)))
        assert ey <= (1e-4 if dtype == torch.float32 else TOL_BF16_OUT) and es <= tol, s


# ------------------------------------------------------- full-size workloads
def test_prefill_t4096_h8_full(dev):
    w = W.WORKLOADS["prefill_t4096_h8"]
    say("prefill_t4096_h8: B=1 H=8 T=4096, full oracle comparison")
    x = W.prefill_inputs(w, seed=0)
    out, fin = run_gpu(x, dev)
    ro, rf = run_oracle(x)
    check(out, fin, ro, rf, TOL_BF16_OUT, TOL_BF16_STATE, "prefill_t4096_h8")
    log_worst("prefill_t4096_h8", out, ro, fin, rf)


def test_varlen_4seq_h32_full(dev):
    w = W.WORKLOADS["varlen_4seq_h32"]
    say(f"varlen_4seq_h32: lengths {W.varlen_lengths(w, 0)}, full oracle comparison")
    x = W.prefill_inputs(w, seed=0, device=dev)
    out, fin = run_gpu(x, dev)
    ro, rf = run_oracle(x)
    check(out, fin, ro, rf, TOL_BF16_OUT, TOL_BF16_STATE, "varlen_4seq_h32")
    log_worst("varlen_4seq_h32", out, ro, fin, rf, cu=x["cu_seqlens"].cpu().numpy())


def test_decode_n256_h32_full(dev):
    w = W.WORKLOADS["decode_n256_h32"]
    say("decode_n256_h32: N=256 H=32, 128 steps, zero init, oracle every step")
    st = W.decode_init_state(w, device=dev)
    st64 = np.zeros(tuple(st.shape), dtype=np.float64)
    worst, worst_nh = 0.0, (0.0, (0, 0), 0)
    for s in range(w.steps):
        x = W.decode_inputs(w, step=s, device=dev)
        y = kda.decode_step(x["q"], x["k"], x["v"], x["g"], x["beta"], x["z"], st)
        ry = oracle.decode_step(np32(x["q"]), np32(x["k"]), np32(x["v"]), np32(x["g"]),
                                np32(x["beta"]), np32(x["z"]), st64)
        worst = max(worst, rel(np32(y), ry))
        # outputs [N, H, dv] as one-token sequences: slice per (n, h)
        e, nh = worst_slice(np32(y)[:, None], ry[:, None], "out")
        if e > worst_nh[0]:
            worst_nh = (e, nh, s)
    es = rel(np32(st), st64)
    ess, nhs = worst_slice(np32(st), st64, "state")
    say(f"decode_n256_h32: worst step out rel err {worst:.3e}, final state rel err {es:.3e}")
    say(f"decode_n256_h32: worst (n, h) out slice {worst_nh[1]} at step {worst_nh[2]} rel err "
        f"{worst_nh[0]:.3e}; worst state slice {nhs} rel err {ess:.3e}")
    assert worst <= TOL_BF16_OUT and es <= TOL_BF16_STATE


def test_long_t1m_h16_all_heads(dev):
    """The 1M-token workload: the full call, and the split at T/2 whose second
    half starts from the first half's final state, which must equal the
    single call bitwise.  Every one of the 16 heads is compared with the
    oracle over all 2^20 tokens: the oracle streams each half per head and
    keeps only per-head maxima (no float64 output array), and the tolerances
    hold per head, not only over the whole tensor."""
    w = W.WORKLOADS["long_t1m_h16"]
    T, H = w.T, w.H
    say("long_t1m_h16: T=1048576 H=16, pinned quarter of channels at g=-5; full call, "
        "split at T/2, oracle on all 16 heads")
    x = W.prefill_inputs(w, seed=0, device=dev)
    out, fin = run_gpu(x, dev)
    half = T // 2
    keys = ("q", "k", "v", "g", "beta", "z")
    a = {k: x[k][:, :half].contiguous() for k in keys}
    o1, s1 = kda.chunk_fwd(a["q"], a["k"], a["v"], a["g"], a["beta"], a["z"])
    del a
    b = {k: x[k][:, half:].contiguous() for k in keys}
    o2, s2 = kda.chunk_fwd(b["q"], b["k"], b["v"], b["g"], b["beta"], b["z"], init_state=s1)
    torch.cuda.synchronize()
    del b
    # T/2 is a multiple of the chunk: the split call does identical arithmetic
    assert torch.equal(o1, out[:, :half]) and torch.equal(o2, out[:, half:])
    assert torch.equal(s2, fin)
    del o1, o2
    bits = lambda t: t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    xb = {k: bits(x[k]) for k in keys}
    ob = bits(out)
    del x, out
    threads = max(1, min(os.cpu_count() or 1, 16))
    say(f"long_t1m_h16: oracle over the first half ({threads} threads)")
    e1, r1, mid = oracle.forward_compare(*(xb[k][:, :half] for k in keys), ob[:, :half],
                                         bf16=True, n_threads=threads)
    say("long_t1m_h16: oracle over the second half from its exact state at T/2")
    e2, r2, ref_fin = oracle.forward_compare(*(xb[k][:, half:] for k in keys), ob[:, half:],
                                             init_state=mid, bf16=True, n_threads=threads)
    s1n, finn = np32(s1), np32(fin)
    out_rel = np.maximum(e1[0], e2[0]) / np.maximum(np.maximum(r1[0], r2[0]), 1e-30)
    mid_rel = np.array([rel(s1n[0, h], mid[0, h]) for h in range(H)])
    fin_rel = np.array([rel(finn[0, h], ref_fin[0, h]) for h in range(H)])
    for h in range(H):
        say(f"long_t1m_h16 head {h:2d}: out rel err {out_rel[h]:.3e}, state at T/2 "
            f"{mid_rel[h]:.3e}, final state {fin_rel[h]:.3e}")
    whole = max(e1.max(), e2.max()) / max(r1.max(), r2.max())
    say(f"long_t1m_h16: whole-tensor out rel err {whole:.3e}; worst head out "
        f"{int(out_rel.argmax())} ({out_rel.max():.3e}), state at T/2 {int(mid_rel.argmax())} "
        f"({mid_rel.max():.3e}), final {int(fin_rel.argmax())} ({fin_rel.max():.3e})")
    assert np.all(out_rel <= TOL_BF16_OUT), out_rel
    assert np.all(mid_rel <= TOL_BF16_STATE), mid_rel
    assert np.all(fin_rel <= TOL_BF16_STATE), fin_rel
