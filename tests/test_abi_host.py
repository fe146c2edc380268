"""Host-only checks of the C ABI: the library loads, exports every function
``include/kda.h`` declares, sizes its workspace as documented and rejects bad
arguments with the documented status codes before launching anything (no
GPU is touched by these calls)."""
from __future__ import annotations

import ctypes
import os
import re

import pytest

import kimi_delta_attention_chunkwise_amd as kda

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kda.h")

OK, NULLP, SHAPE, DTYPE, UNSUP, WS, HIP, MISAL, SCRATCH = range(9)
A = 1 << 20            # a fake device address with every alignment


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kda_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(kda.library_path()):
        pytest.skip("libkda.so not built")
    return kda.load_library()


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("kda_chunk_fwd", "kda_decode_step", "kda_chunk_fwd_workspace_bytes",
              "kda_status_str", "kda_chunk_fwd_snapshots", "kda_snapshot_slots",
              "kda_chunk_fwd_ex", "kda_decode_step_ex", "kda_decode_verify",
              "kda_decode_commit", "kda_chunk_bwd", "kda_chunk_bwd_workspace_bytes",
              "kda_chunk_bwd_ex", "kda_chunk_fwd_noalloc",
              "kda_chunk_bwd_supported"):
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    missing = [n for n in declared_functions() if not hasattr(lib, n)]
    assert not missing, missing


def test_status_strings(lib):
    for code, name in enumerate(["KDA_OK", "KDA_ERR_NULL_POINTER", "KDA_ERR_BAD_SHAPE",
                                 "KDA_ERR_BAD_DTYPE", "KDA_ERR_UNSUPPORTED",
                                 "KDA_ERR_WORKSPACE_TOO_SMALL", "KDA_ERR_HIP",
                                 "KDA_ERR_MISALIGNED", "KDA_ERR_SCRATCH_LIMIT"]):
        assert lib.kda_status_str(code).decode() == name
    assert lib.kda_status_str(99).decode() == "KDA_ERR_UNKNOWN"


def test_supported_sets(lib):
    assert lib.kda_chunk_fwd_supported(1, 128, 128, 64) == 1
    assert lib.kda_chunk_fwd_supported(0, 16, 16, 16) == 1
    for args in [(1, 128, 128, 16), (1, 64, 64, 64), (0, 128, 128, 64), (0, 16, 16, 64),
                 (2, 128, 128, 64)]:
        assert lib.kda_chunk_fwd_supported(*args) == 0
    for dt in (0, 1):
        for d in (16, 128):
            assert lib.kda_decode_step_supported(dt, d, d) == 1
    assert lib.kda_decode_step_supported(1, 64, 64) == 0
    assert lib.kda_decode_step_supported(1, 128, 16) == 0


def test_workspace_bytes(lib):
    ws = lib.kda_chunk_fwd_workspace_bytes
    rb = lib.kda_chunk_fwd_records_bytes
    PREC = ws(1, 64, 1, 1, 128, 128, 64, 1, 0)      # one pair slot (here holding one chunk)
    REC = rb(1, 64, 1, 1, 128, 128, 64, 1, 0)       # one 64-token chunk of one head
    assert PREC % 256 == 0 and REC % 256 == 0
    # bytes per token-head as documented: pair records 1,284, chunk records 2,824
    assert PREC == 164352 and PREC // 128 == 1284
    assert REC == 180736 and REC // 64 == 2824
    # fixed length: B * ceil(T / 128) pair slots per head
    assert ws(1, 4096, 1, 8, 128, 128, 64, 1, 0) == 32 * 8 * PREC
    assert ws(3, 100, 3, 2, 128, 128, 64, 1, 0) == 3 * 2 * 1 * PREC
    assert ws(3, 200, 3, 2, 128, 128, 64, 1, 0) == 3 * 2 * 2 * PREC
    assert ws(1, 0, 1, 4, 128, 128, 64, 1, 0) == 0
    # varlen: floor(T / 128) + N pair slots per head
    assert ws(1, 67000, 4, 32, 128, 128, 64, 1, 1) == (67000 // 128 + 4) * 32 * PREC
    # the 1M-token workload: 8,192 pairs x 16 heads, 21.5 GB (per-chunk records: 47.4 GB)
    assert ws(1, 1 << 20, 1, 16, 128, 128, 64, 1, 0) == 8192 * 16 * PREC
    assert ws(1, 1 << 20, 1, 16, 128, 128, 64, 1, 0) < 24e9
    # per-chunk records: B * ceil(T / 64), or floor(T / 64) + N, chunk slots per head
    assert rb(1, 4096, 1, 8, 128, 128, 64, 1, 0) == 64 * 8 * REC
    assert rb(3, 100, 3, 2, 128, 128, 64, 1, 0) == 3 * 2 * 2 * REC
    assert rb(1, 67000, 4, 32, 128, 128, 64, 1, 1) == (67000 // 64 + 4) * 32 * REC
    # fp32 path needs none
    assert ws(1, 64, 1, 2, 16, 16, 16, 0, 0) == 0 and rb(1, 64, 1, 2, 16, 16, 16, 0, 0) == 0
    bad = ctypes.c_size_t(-1).value
    for fn in (ws, rb):
        assert fn(1, 64, 1, 2, 64, 64, 64, 1, 0) == bad           # unsupported dims
        assert fn(2, 64, 1, 2, 128, 128, 64, 1, 1) == bad         # varlen needs B = 1
        assert fn(2, 64, 3, 2, 128, 128, 64, 1, 0) == bad         # N must equal B


def test_chunk_records_flag_needs_the_records_size(lib):
    """KDA_FWD_CHUNK_RECORDS keeps one record per chunk: a workspace of the
    pair-record size is too small for it (T = 4096: 64 chunk records of
    180,736 B against 32 pair records of 164,352 B)."""
    p = ctypes.c_void_p
    PREC_ALL = lib.kda_chunk_fwd_workspace_bytes(1, 4096, 1, 1, 128, 128, 64, 1, 0)
    REC_ALL = lib.kda_chunk_fwd_records_bytes(1, 4096, 1, 1, 128, 128, 64, 1, 0)
    assert REC_ALL > PREC_ALL

    def chunk(flags, nbytes):
        return lib.kda_chunk_fwd_ex(p(1), p(1), p(1), p(1), p(1), p(1), None, p(1), None, None, 0,
                                    None, 1, 4096, 1, 1, 128, 128, 64, 1.0, 1, flags, p(1), nbytes,
                                    None)
    assert chunk(kda.FWD_CHUNK_RECORDS, PREC_ALL) == WS
    assert chunk(kda.FWD_CHUNK_RECORDS, REC_ALL - 1) == WS
    assert chunk(0, PREC_ALL - 1) == WS
    # enough bytes: the next check (the misaligned fake pointers) answers
    assert chunk(kda.FWD_CHUNK_RECORDS, REC_ALL) == MISAL
    assert chunk(0, PREC_ALL) == MISAL


def _chunk(lib, **kw):
    a = dict(q=1, k=1, v=1, g=1, beta=1, gate=1, init=None, out=1, final=None, cu=None,
             B=1, T=64, N=1, H=2, dk=128, dv=128, chunk=64, scale=1.0, dt=1, ws=None,
             ws_bytes=0)
    a.update(kw)
    p = lambda x: None if x is None else ctypes.c_void_p(x)
    return lib.kda_chunk_fwd(p(a["q"]), p(a["k"]), p(a["v"]), p(a["g"]), p(a["beta"]),
                             p(a["gate"]), p(a["init"]), p(a["out"]), p(a["final"]), p(a["cu"]),
                             a["B"], a["T"], a["N"], a["H"], a["dk"], a["dv"], a["chunk"],
                             a["scale"], a["dt"], p(a["ws"]), a["ws_bytes"], None)


def test_chunk_fwd_rejects_bad_arguments_before_launch(lib):
    REC = lib.kda_chunk_fwd_workspace_bytes(1, 64, 1, 1, 128, 128, 64, 1, 0)
    assert _chunk(lib, dt=7) == DTYPE
    assert _chunk(lib, dk=64, dv=64) == UNSUP
    assert _chunk(lib, chunk=16) == UNSUP
    assert _chunk(lib, H=0) == SHAPE
    assert _chunk(lib, T=-1) == SHAPE
    assert _chunk(lib, B=2, N=1) == SHAPE
    assert _chunk(lib, B=2, N=2, cu=1) == SHAPE               # varlen needs B = 1
    assert _chunk(lib, q=None, ws=1, ws_bytes=10 ** 9) == NULLP
    assert _chunk(lib, gate=None, ws=1, ws_bytes=10 ** 9) == NULLP
    assert _chunk(lib, ws=None, ws_bytes=0) == NULLP          # bf16 needs a workspace
    assert _chunk(lib, ws=1, ws_bytes=REC) == WS              # 2 heads need 2 records
    # nothing to do: zero sequences
    assert _chunk(lib, cu=1, N=0, T=0, q=None, k=None, v=None, g=None, beta=None, gate=None,
                  out=None) == OK


def test_misaligned_pointers_are_rejected_before_launch(lib):
    """Tensors need 16 bytes, beta its element, cu_seqlens 4 bytes and the
    workspace 256; each case has exactly one pointer below its alignment."""
    REC = lib.kda_chunk_fwd_workspace_bytes(1, 64, 1, 2, 128, 128, 64, 1, 0)
    ok = dict(q=A, k=A, v=A, g=A, beta=A, gate=A, out=A, ws=A, ws_bytes=REC)
    for name, off in [("q", 8), ("k", 2), ("v", 4), ("g", 8), ("gate", 8), ("out", 8),
                      ("init", 8), ("final", 4), ("beta", 1), ("ws", 128)]:
        kw = dict(ok, init=A, final=A)
        kw[name] = A + off
        assert _chunk(lib, **kw) == MISAL, name
    assert _chunk(lib, **dict(ok, cu=A + 2, ws_bytes=4 * REC)) == MISAL
    # checked after the other arguments
    assert _chunk(lib, **dict(ok, q=A + 8, ws_bytes=REC - 1)) == WS
    p = ctypes.c_void_p

    def step(**kw):
        a = dict(q=A, k=A, v=A, g=A, beta=A, gate=A, state=A, out=A)
        a.update(kw)
        return lib.kda_decode_step(*[p(a[n]) for n in ("q", "k", "v", "g", "beta", "gate",
                                                        "state", "out")],
                                   4, 2, 128, 128, 1.0, 1, None)
    for name, off in [("q", 8), ("v", 8), ("gate", 8), ("state", 8), ("out", 2), ("beta", 1)]:
        assert step(**{name: A + off}) == MISAL, name
    assert lib.kda_decode_commit(p(A), p(A), p(A), p(A + 2), p(A), 2, 3, 1, 128, 128, 1, 0,
                                 None) == MISAL
    assert lib.kda_decode_verify(p(A), p(A), p(A), p(A), p(A), p(A), p(A), p(A), p(A + 8), 2, 3,
                                 1, 128, 128, 1.0, 1, 0, None) == MISAL


def test_snapshot_slots(lib):
    slots = lib.kda_snapshot_slots
    bad = ctypes.c_size_t(-1).value
    assert slots(2, 700, 2, 64, 128, 0) == 2 * 5
    assert slots(1, 1000, 3, 64, 128, 1) == 1000 // 128 + 3
    assert slots(1, 0, 0, 64, 64, 1) == 0
    assert slots(1, 64, 1, 64, 100, 0) == bad          # not a multiple of the chunk
    assert slots(1, 64, 1, 64, 32, 0) == bad           # shorter than a chunk
    assert slots(2, 64, 1, 64, 64, 1) == bad           # varlen needs B = 1
    assert slots(2, 64, 3, 64, 64, 0) == bad           # N must equal B


def test_snapshot_index_matches_the_documented_slots():
    # varlen: floor(cu[n] / I) + n + m - 1; fixed: n * floor(T / I) + m - 1
    idx = kda.snapshot_index([300, 0, 256, 700], 128, True)
    assert idx == [(0, 128, 0), (0, 256, 1), (2, 128, 4), (2, 256, 5), (3, 128, 7),
                   (3, 256, 8), (3, 384, 9), (3, 512, 10), (3, 640, 11)]
    assert max(s for _, _, s in idx) < 1256 // 128 + 4
    idx = kda.snapshot_index([700, 700], 192, False, 700)
    assert idx == [(0, 192, 0), (0, 384, 1), (0, 576, 2), (1, 192, 3), (1, 384, 4), (1, 576, 5)]


def test_chunk_fwd_snapshots_rejects_bad_arguments(lib):
    PREC = lib.kda_chunk_fwd_workspace_bytes(1, 256, 1, 1, 128, 128, 64, 1, 0)
    REC = lib.kda_chunk_fwd_records_bytes(1, 256, 1, 1, 128, 128, 64, 1, 0)
    p = lambda x: None if x is None else ctypes.c_void_p(x)

    def call(snaps, interval, **kw):
        a = dict(B=1, T=256, N=1, H=1, ws=1, ws_bytes=REC)
        a.update(kw)
        return lib.kda_chunk_fwd_snapshots(p(1), p(1), p(1), p(1), p(1), p(1), None, p(1), None,
                                           p(snaps), interval, None, a["B"], a["T"], a["N"],
                                           a["H"], 128, 128, 64, 1.0, 1, p(a["ws"]),
                                           a["ws_bytes"], None)
    assert call(1, 100) == SHAPE
    assert call(1, 0) == SHAPE
    # an interval of 64 or 192 tokens falls inside a pair of chunks: per-chunk
    # records (4 x 180,736 B here); multiples of 128 need the pair records
    assert REC > PREC
    assert call(1, 64, ws_bytes=REC - 1) == WS
    assert call(1, 192, ws_bytes=PREC) == WS
    assert call(1, 128, ws_bytes=PREC - 1) == WS
    assert call(1, 128, ws_bytes=PREC) == MISAL      # enough: the fake pointers answer
    assert call(1, 64, B=2) == SHAPE


def test_prologue_rejects_unknown_bits(lib):
    p = ctypes.c_void_p
    REC = lib.kda_chunk_fwd_workspace_bytes(1, 64, 1, 1, 128, 128, 64, 1, 0)

    def chunk(pro):
        return lib.kda_chunk_fwd_ex(p(1), p(1), p(1), p(1), p(1), p(1), None, p(1), None, None, 0,
                                    None, 1, 64, 1, 1, 128, 128, 64, 1.0, 1, pro, p(1), REC, None)

    def dec(pro):
        return lib.kda_decode_step_ex(p(1), p(1), p(1), p(1), p(1), p(1), p(1), p(1), 1, 1, 128,
                                      128, 1.0, 1, pro, None)
    assert chunk(8) == UNSUP and chunk(0xFFFF) == UNSUP and chunk(512) == UNSUP
    assert dec(8) == UNSUP and dec(kda.FWD_CHUNK_RECORDS) == UNSUP


def test_verify_and_commit_reject_bad_arguments(lib):
    p = ctypes.c_void_p

    def verify(**kw):
        a = dict(N=2, K=3, H=1, d=128, dt=1, pro=0, state=1, out=1)
        a.update(kw)
        ptr = lambda x: None if x is None else p(x)
        return lib.kda_decode_verify(p(1), p(1), p(1), p(1), p(1), p(1), ptr(a["state"]),
                                     ptr(a["out"]), None, a["N"], a["K"], a["H"], a["d"], a["d"],
                                     1.0, a["dt"], a["pro"], None)

    def commit(**kw):
        a = dict(N=2, K=3, H=1, d=128, dt=1, pro=0, acc=1, state=1)
        a.update(kw)
        ptr = lambda x: None if x is None else p(x)
        return lib.kda_decode_commit(p(1), p(1), p(1), ptr(a["acc"]), ptr(a["state"]), a["N"],
                                     a["K"], a["H"], a["d"], a["d"], a["dt"], a["pro"], None)
    assert verify(K=0) == SHAPE and commit(K=0) == SHAPE
    assert verify(H=0) == SHAPE and commit(N=-1) == SHAPE
    assert verify(dt=9) == DTYPE and commit(dt=9) == DTYPE
    assert verify(d=64) == UNSUP and commit(d=64) == UNSUP
    assert verify(pro=16) == UNSUP and commit(pro=16) == UNSUP
    assert verify(state=None) == NULLP and verify(out=None) == NULLP
    assert commit(acc=None) == NULLP and commit(state=None) == NULLP
    assert verify(N=0) == OK and commit(N=0) == OK


def test_decode_step_rejects_bad_arguments_before_launch(lib):
    p = ctypes.c_void_p

    def call(**kw):
        a = dict(q=1, k=1, v=1, g=1, beta=1, gate=1, state=1, out=1, N=4, H=2, dk=128, dv=128,
                 scale=1.0, dt=1)
        a.update(kw)
        ptr = lambda x: None if x is None else p(x)
        return lib.kda_decode_step(ptr(a["q"]), ptr(a["k"]), ptr(a["v"]), ptr(a["g"]),
                                   ptr(a["beta"]), ptr(a["gate"]), ptr(a["state"]), ptr(a["out"]),
                                   a["N"], a["H"], a["dk"], a["dv"], a["scale"], a["dt"], None)
    assert call(dt=5) == DTYPE
    assert call(dk=64, dv=64) == UNSUP
    assert call(N=-1) == SHAPE
    assert call(H=0) == SHAPE
    assert call(state=None) == NULLP
    assert call(out=None) == NULLP
    assert call(N=0, q=None) == OK


def test_chunk_bwd_sizes_and_argument_checks(lib):
    assert lib.kda_chunk_bwd_supported(0, 16, 16, 16) == 1
    assert lib.kda_chunk_bwd_supported(1, 128, 128, 64) == 1
    for args in [(1, 128, 128, 16), (0, 16, 16, 64), (0, 128, 128, 16), (2, 16, 16, 16)]:
        assert lib.kda_chunk_bwd_supported(*args) == 0
    ws = lib.kda_chunk_bwd_workspace_bytes
    bad = ctypes.c_size_t(-1).value
    # one fp32 16 x 16 entry state per (16-token chunk slot, head)
    assert ws(2, 37, 2, 3, 16, 16, 16, 0, 0) == 2 * 3 * 3 * 1024
    assert ws(1, 55, 5, 2, 16, 16, 16, 0, 1) == (55 // 16 + 5) * 2 * 1024
    assert ws(1, 0, 1, 2, 16, 16, 16, 0, 0) == 0
    assert ws(2, 64, 1, 1, 16, 16, 16, 0, 0) == bad
    # bf16: a forward and a backward record per (64-token chunk slot, head)
    REC = lib.kda_chunk_fwd_records_bytes(1, 64, 1, 1, 128, 128, 64, 1, 0)
    assert ws(1, 4096, 1, 8, 128, 128, 64, 1, 0) == 2 * 64 * 8 * REC
    assert ws(1, 1000, 3, 2, 128, 128, 64, 1, 1) == 2 * (1000 // 64 + 3) * 2 * REC
    assert ws(1, 64, 1, 1, 128, 128, 16, 1, 0) == bad
    p = lambda x: None if x is None else ctypes.c_void_p(x)

    def call(**kw):
        a = dict(q=1, gq=1, B=1, T=64, N=1, H=2, d=16, chunk=16, dt=0, cu=None, ws=1,
                 ws_bytes=10 ** 9)
        a.update(kw)
        return lib.kda_chunk_bwd(p(a["q"]), p(1), p(1), p(1), p(1), p(1), None, p(1), None,
                                 p(a["gq"]), p(1), p(1), p(1), p(1), p(1), None, p(a["cu"]),
                                 a["B"], a["T"], a["N"], a["H"], a["d"], a["d"], a["chunk"], 1.0,
                                 a["dt"], p(a["ws"]), a["ws_bytes"], None)
    assert call(dt=4) == DTYPE
    assert call(dt=1, d=128, chunk=16) == UNSUP
    assert call(chunk=64) == UNSUP
    assert call(dt=1, d=128, chunk=64, ws_bytes=REC) == WS
    assert call(H=0) == SHAPE and call(T=-1) == SHAPE and call(B=2) == SHAPE
    assert call(cu=1, B=2, N=2) == SHAPE
    assert call(q=None) == NULLP and call(gq=None) == NULLP
    assert call(ws=None) == NULLP
    assert call(ws_bytes=2 * 4 * 1024 - 1) == WS
    assert call(cu=1, N=0, T=0, q=None, gq=None) == OK

    def call_ex(fwd, fwd_bytes, ws_bytes, dt=1, d=128, chunk=64):
        return lib.kda_chunk_bwd_ex(p(1), p(1), p(1), p(1), p(1), p(1), None, p(1), None,
                                    p(1), p(1), p(1), p(1), p(1), p(1), None, None, 1, 64, 1, 2,
                                    d, d, chunk, 1.0, dt, p(fwd), fwd_bytes, p(1), ws_bytes, None)
    # (only calls that fail validation: nothing may launch with these fake pointers)
    # H = 2: a record array is 2 REC; the backward alone needs two arrays, with the
    # forward's records one array
    assert call_ex(None, 0, 4 * REC - 1) == WS
    assert call_ex(1, 2 * REC - 1, 10 ** 9) == WS           # forward records too small
    assert call_ex(1, 2 * REC, 2 * REC - 1) == WS           # below one record array
    assert call_ex(1, 10 ** 9, 10 ** 9, dt=0, d=16, chunk=16) == UNSUP   # fp32 keeps no records


def test_python_binding_refuses_cpu_tensors(lib):
    import torch
    q = torch.zeros(1, 4, 1, 16)
    with pytest.raises(ValueError):
        kda.chunk_fwd(q, q, q, q, torch.zeros(1, 4, 1), q)
    st = torch.zeros(1, 1, 16, 16)
    with pytest.raises(ValueError):
        kda.decode_step(q[0], q[0], q[0], q[0], torch.zeros(1, 1), q[0], st)


def test_missing_library_fails_loudly(tmp_path):
    with pytest.raises(kda.KdaLibraryError):
        kda.load_library(str(tmp_path / "nope.so"))


def test_noalloc_rejects_sizes_beyond_its_scratch(lib):
    """kda_chunk_fwd_noalloc checks its workspace need against the static
    scratch size before touching the device; argument errors come first."""
    ws = lib.kda_chunk_fwd_workspace_bytes
    rec = ws(1, 128, 1, 1, 128, 128, 64, 1, 0)         # one pair record
    limit = kda.NOALLOC_SCRATCH_BYTES
    H = 8
    t_fit = (limit // (rec * H)) * 128          # the longest B=1, H=8 call that fits
    assert ws(1, t_fit, 1, H, 128, 128, 64, 1, 0) <= limit
    assert ws(1, t_fit + 1, 1, H, 128, 128, 64, 1, 0) > limit
    fn = lib.kda_chunk_fwd_noalloc
    p = [ctypes.c_void_p(A)] * 6
    assert fn(*p, None, ctypes.c_void_p(A), None, None, 1, t_fit + 1, 1, H, 128, 128, 64,
              1.0, 1, None) == SCRATCH
    # unsupported sizes and bad shapes are reported as such, not as the limit
    assert fn(*p, None, ctypes.c_void_p(A), None, None, 1, 64, 1, H, 64, 64, 64, 1.0, 1,
              None) == UNSUP
    assert fn(*p, None, ctypes.c_void_p(A), None, None, 2, 64, 1, H, 128, 128, 64, 1.0, 1,
              None) == SHAPE
    assert fn(None, *p[1:], None, ctypes.c_void_p(A), None, None, 1, 64, 1, H, 128, 128, 64,
              1.0, 1, None) == NULLP
    # without cu_seqlens N must equal B
    assert fn(*p, None, ctypes.c_void_p(A), None, None, 1, 64, 0, H, 128, 128, 64, 1.0, 1,
              None) == SHAPE
