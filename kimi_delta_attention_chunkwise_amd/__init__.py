"""Kimi Delta Attention (KDA) for MI355X (gfx950): Python binding of libkda.so.

The binding only marshals arguments: it checks tensor shapes, dtypes and
devices, allocates outputs and the workspace with PyTorch, and calls the C ABI
declared in ``include/kda.h`` on the current HIP stream.  Every step of the
computation runs in the HIP kernels of ``libkda.so``; there is no fallback.
If the library is missing the calls raise ``KdaLibraryError``.

Entry points (names follow the C ABI):
  chunk_fwd(q, k, v, g, beta, gate, init_state=None, output_final_state=True,
            cu_seqlens=None, chunk=None, scale=1.0) -> (out, final_state)
  chunk_fwd_snapshots(q, k, v, g, beta, gate, interval, ...)
            -> (out, final_state, snapshots)
  chunk_fwd_noalloc(q, k, v, g, beta, gate, ...) -> (out, final_state)
            (no workspace: the library's static scratch array)
  decode_step(q, k, v, g, beta, gate, state, scale=1.0) -> out   (state in place)
  decode_verify(q, k, v, g, beta, gate, state, ...) -> (out, u)  (K draft tokens, state kept)
  decode_commit(k, g, u, accepted, state, ...)                   (accepted prefix into state)
  chunk_bwd(q, k, v, g, beta, gate, grad_out, init_state=None, grad_final_state=None, ...)
            -> dict of gradients (training backward)
  chunk_fwd_workspace_bytes(...), chunk_bwd_workspace_bytes(...), snapshot_slots(...),
  chunk_fwd_supported(...), chunk_bwd_supported(...), decode_step_supported(...)
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = [
    "KdaError", "KdaLibraryError", "chunk_fwd", "chunk_fwd_snapshots", "decode_step",
    "decode_verify", "decode_commit", "chunk_bwd", "chunk_bwd_workspace_bytes",
    "chunk_bwd_supported", "chunk_fwd_workspace_bytes", "snapshot_slots", "snapshot_index",
    "chunk_fwd_supported", "decode_step_supported", "library_path", "load_library",
    "KDA_F32", "KDA_BF16", "G_MIN", "PRO_QK_L2NORM", "PRO_BETA_SIGMOID", "PRO_G_SOFTPLUS",
    "chunk_fwd_noalloc", "NOALLOC_SCRATCH_BYTES", "FWD_CHUNK_RECORDS",
]

KDA_F32 = 0
KDA_BF16 = 1
G_MIN = -5.0
# prologue bits (KDA_PRO_* in kda.h)
PRO_QK_L2NORM = 1
PRO_BETA_SIGMOID = 2
PRO_G_SOFTPLUS = 4
# forward flag: keep per-chunk records for the backward (KDA_FWD_CHUNK_RECORDS)
FWD_CHUNK_RECORDS = 256
_DEFAULT_CHUNK = {KDA_F32: 16, KDA_BF16: 64}

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_NAME = "libkda.so"
_lib = None


class KdaError(RuntimeError):
    """A libkda call returned an error status."""


class KdaLibraryError(ImportError):
    """libkda.so is missing or cannot be loaded."""


def library_path() -> str:
    return os.path.join(_PKG, _LIB_NAME)


_SIGNATURES = {
    "kda_status_str": ([ctypes.c_int], ctypes.c_char_p),
    "kda_chunk_fwd_supported": ([ctypes.c_int] * 4, ctypes.c_int),
    "kda_decode_step_supported": ([ctypes.c_int] * 3, ctypes.c_int),
    "kda_chunk_fwd_workspace_bytes": ([ctypes.c_int] * 9, ctypes.c_size_t),
    "kda_chunk_fwd_records_bytes": ([ctypes.c_int] * 9, ctypes.c_size_t),
    "kda_chunk_fwd": ([ctypes.c_void_p] * 10 + [ctypes.c_int] * 7 + [ctypes.c_float, ctypes.c_int,
                      ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p], ctypes.c_int),
    "kda_snapshot_slots": ([ctypes.c_int] * 6, ctypes.c_size_t),
    "kda_chunk_fwd_snapshots": ([ctypes.c_void_p] * 10 + [ctypes.c_int] + [ctypes.c_void_p]
                                + [ctypes.c_int] * 7 + [ctypes.c_float, ctypes.c_int,
                                ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p], ctypes.c_int),
    "kda_chunk_fwd_ex": ([ctypes.c_void_p] * 10 + [ctypes.c_int] + [ctypes.c_void_p]
                         + [ctypes.c_int] * 7 + [ctypes.c_float, ctypes.c_int, ctypes.c_uint,
                         ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p], ctypes.c_int),
    "kda_decode_step_ex": ([ctypes.c_void_p] * 8 + [ctypes.c_int] * 4 + [ctypes.c_float, ctypes.c_int,
                           ctypes.c_uint, ctypes.c_void_p], ctypes.c_int),
    "kda_decode_verify": ([ctypes.c_void_p] * 9 + [ctypes.c_int] * 5 + [ctypes.c_float,
                          ctypes.c_int, ctypes.c_uint, ctypes.c_void_p], ctypes.c_int),
    "kda_decode_commit": ([ctypes.c_void_p] * 5 + [ctypes.c_int] * 5 + [ctypes.c_int, ctypes.c_uint,
                          ctypes.c_void_p], ctypes.c_int),
    "kda_chunk_bwd_supported": ([ctypes.c_int] * 4, ctypes.c_int),
    "kda_chunk_bwd_workspace_bytes": ([ctypes.c_int] * 9, ctypes.c_size_t),
    "kda_chunk_bwd": ([ctypes.c_void_p] * 17 + [ctypes.c_int] * 7 + [ctypes.c_float, ctypes.c_int,
                      ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p], ctypes.c_int),
    "kda_chunk_bwd_ex": ([ctypes.c_void_p] * 17 + [ctypes.c_int] * 7 + [ctypes.c_float, ctypes.c_int,
                         ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_size_t,
                         ctypes.c_void_p], ctypes.c_int),
    "kda_decode_step": ([ctypes.c_void_p] * 8 + [ctypes.c_int] * 4 + [ctypes.c_float, ctypes.c_int,
                        ctypes.c_void_p], ctypes.c_int),
    "kda_chunk_fwd_noalloc": ([ctypes.c_void_p] * 10 + [ctypes.c_int] * 7 + [ctypes.c_float,
                              ctypes.c_int, ctypes.c_void_p], ctypes.c_int),
}

# size of the static scratch array of kda_chunk_fwd_noalloc (KDA_NOALLOC_SCRATCH_BYTES)
NOALLOC_SCRATCH_BYTES = 128 << 20


def load_library(path: str | None = None):
    """Load libkda.so (once) and declare its C signatures."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or library_path()
    if not os.path.exists(p):
        raise KdaLibraryError(
            f"{p} not found: build it with `python -m kimi_delta_attention_chunkwise_amd._build`")
    try:
        lib = ctypes.CDLL(p)
    except OSError as exc:  # pragma: no cover - depends on the loader
        raise KdaLibraryError(f"cannot load {p}: {exc}") from exc
    for name, (argtypes, restype) in _SIGNATURES.items():
        fn = getattr(lib, name)
        fn.argtypes = argtypes
        fn.restype = restype
    if path is None:
        _lib = lib
    return lib


def _check(status: int):
    if status != 0:
        msg = load_library().kda_status_str(status).decode()
        raise KdaError(f"libkda returned {msg} ({status})")


def _dtype_code(t: torch.dtype) -> int:
    if t == torch.float32:
        return KDA_F32
    if t == torch.bfloat16:
        return KDA_BF16
    raise TypeError(f"unsupported dtype {t}; use float32 or bfloat16")


def _ptr(t: torch.Tensor | None):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream_ptr(device: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def chunk_fwd_supported(dtype: torch.dtype, dk: int, dv: int, chunk: int) -> bool:
    return bool(load_library().kda_chunk_fwd_supported(_dtype_code(dtype), dk, dv, chunk))


def decode_step_supported(dtype: torch.dtype, dk: int, dv: int) -> bool:
    return bool(load_library().kda_decode_step_supported(_dtype_code(dtype), dk, dv))


def chunk_fwd_workspace_bytes(B: int, T: int, N: int, H: int, dk: int, dv: int, chunk: int,
                              dtype: torch.dtype, varlen: bool, chunk_records: bool = False) -> int:
    """Workspace bytes of a forward; ``chunk_records``: per-chunk records (a
    forward whose workspace a backward will reuse, or a snapshot interval that
    is an odd multiple of 64), else the pair records of the default forward."""
    lib = load_library()
    fn = lib.kda_chunk_fwd_records_bytes if chunk_records else lib.kda_chunk_fwd_workspace_bytes
    n = fn(B, T, N, H, dk, dv, chunk, _dtype_code(dtype), int(varlen))
    if n == ctypes.c_size_t(-1).value:
        raise KdaError("unsupported or invalid sizes for kda_chunk_fwd")
    return int(n)


def _need(t: torch.Tensor, name: str, shape, dtype, device):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def snapshot_slots(B: int, T: int, N: int, chunk: int, interval: int, varlen: bool) -> int:
    """Number of snapshot slots ``kda_chunk_fwd_snapshots`` indexes for these sizes."""
    n = load_library().kda_snapshot_slots(B, T, N, chunk, interval, int(varlen))
    if n == ctypes.c_size_t(-1).value:
        raise KdaError("invalid sizes or snapshot interval")
    return int(n)


def snapshot_index(lengths, interval: int, varlen: bool, T: int | None = None):
    """Host-side map of the snapshot slots: a list of (sequence n, tokens m *
    interval, slot) for every snapshot the library writes.  ``lengths`` are the
    sequence lengths (for varlen, in packing order); ``T`` is the common
    length when not varlen."""
    res = []
    start = 0
    for n, ln in enumerate(lengths):
        base = (start // interval + n) if varlen else n * (T // interval)
        for m in range(1, ln // interval + 1):
            res.append((n, m * interval, base + m - 1))
        start += ln
    return res


def _chunk_call(q, k, v, g, beta, gate, init_state, output_final_state, cu_seqlens, chunk,
                scale, workspace, out, final_state, interval, snapshots, prologue,
                chunk_records=False):
    lib = load_library()
    if q.dim() != 4:
        raise ValueError("q must be [B, T, H, dk]")
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("kda.chunk_fwd runs on a HIP device; tensors are on " + str(dev))
    dt = q.dtype
    code = _dtype_code(dt)
    chunk = _DEFAULT_CHUNK[code] if chunk is None else int(chunk)
    for name, t, shp in (("k", k, (B, T, H, dk)), ("g", g, (B, T, H, dk)),
                         ("v", v, (B, T, H, dv)), ("gate", gate, (B, T, H, dv)),
                         ("beta", beta, (B, T, H))):
        _need(t, name, shp, dt, dev)
    _need(q, "q", (B, T, H, dk), dt, dev)
    if cu_seqlens is not None:
        if cu_seqlens.dtype != torch.int32 or cu_seqlens.dim() != 1:
            raise TypeError("cu_seqlens must be a 1-D int32 tensor")
        _need(cu_seqlens, "cu_seqlens", cu_seqlens.shape, torch.int32, dev)
        if B != 1:
            raise ValueError("cu_seqlens requires B == 1")
        N = cu_seqlens.numel() - 1
    else:
        N = B
    if init_state is not None:
        _need(init_state, "init_state", (N, H, dk, dv), torch.float32, dev)
    if out is None:
        out = torch.empty((B, T, H, dv), dtype=dt, device=dev)
    else:
        _need(out, "out", (B, T, H, dv), dt, dev)
    if output_final_state:
        if final_state is None:
            final_state = torch.empty((N, H, dk, dv), dtype=torch.float32, device=dev)
        else:
            _need(final_state, "final_state", (N, H, dk, dv), torch.float32, dev)
    else:
        final_state = None
    per_chunk = bool(chunk_records) or (interval is not None and int(interval) % (2 * chunk) != 0)
    nbytes = chunk_fwd_workspace_bytes(B, T, N, H, dk, dv, chunk, dt, cu_seqlens is not None,
                                       per_chunk)
    flags = int(prologue) | (FWD_CHUNK_RECORDS if chunk_records else 0)
    if workspace is None:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)
    elif workspace.device != dev or workspace.dtype != torch.uint8 or workspace.numel() < nbytes:
        raise ValueError(f"workspace must be a uint8 tensor of at least {nbytes} bytes on {dev}")
    if interval is not None:
        slots = snapshot_slots(B, T, N, chunk, int(interval), cu_seqlens is not None)
        if snapshots is None:
            snapshots = torch.empty((slots, H, dk, dv), dtype=torch.float32, device=dev)
        else:
            _need(snapshots, "snapshots", (slots, H, dk, dv), torch.float32, dev)
    if flags:
        st = lib.kda_chunk_fwd_ex(
            _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(gate), _ptr(init_state),
            _ptr(out), _ptr(final_state), _ptr(snapshots), int(interval or 0), _ptr(cu_seqlens),
            B, T, N, H, dk, dv, chunk, float(scale), code, flags, _ptr(workspace),
            workspace.numel(), _stream_ptr(dev))
    elif interval is not None:
        st = lib.kda_chunk_fwd_snapshots(
            _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(gate), _ptr(init_state),
            _ptr(out), _ptr(final_state), _ptr(snapshots), int(interval), _ptr(cu_seqlens),
            B, T, N, H, dk, dv, chunk, float(scale), code, _ptr(workspace), workspace.numel(),
            _stream_ptr(dev))
    else:
        st = lib.kda_chunk_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(gate),
                               _ptr(init_state), _ptr(out), _ptr(final_state), _ptr(cu_seqlens),
                               B, T, N, H, dk, dv, chunk, float(scale), code, _ptr(workspace),
                               workspace.numel(), _stream_ptr(dev))
    _check(st)
    return out, final_state, snapshots


def chunk_fwd(q, k, v, g, beta, gate, init_state=None, output_final_state=True,
              cu_seqlens=None, chunk=None, scale=1.0, workspace=None, out=None,
              final_state=None, prologue=0, chunk_records=False):
    """Chunkwise-parallel KDA forward on the GPU.

    q, k, g ``[B, T, H, dk]``; v, gate ``[B, T, H, dv]``; beta ``[B, T, H]``, all
    of one dtype (bf16 or fp32) on one HIP device.  ``gate`` holds logits.
    ``init_state``: fp32 ``[N, H, dk, dv]`` or None.  ``cu_seqlens``: int32
    ``[N + 1]`` on the device (then B must be 1) or None (N = B).
    Optional preallocated ``workspace`` (uint8, at least
    ``chunk_fwd_workspace_bytes`` bytes), ``out`` and ``final_state``.
    ``prologue``: PRO_* bits for raw inputs (q/k L2 norm, beta logits, g
    pre-activations); 0 for prepared inputs.  ``chunk_records``: keep per-chunk
    records in ``workspace`` (sized by ``chunk_fwd_workspace_bytes(...,
    chunk_records=True)``) for a following ``chunk_bwd(..., fwd_workspace=)``.
    Returns ``(out, final_state)``; final_state is None unless requested.
    """
    out, final_state, _ = _chunk_call(q, k, v, g, beta, gate, init_state, output_final_state,
                                      cu_seqlens, chunk, scale, workspace, out, final_state,
                                      None, None, prologue, chunk_records)
    return out, final_state


def chunk_fwd_noalloc(q, k, v, g, beta, gate, init_state=None, output_final_state=True,
                      cu_seqlens=None, chunk=None, scale=1.0, out=None, final_state=None):
    """``chunk_fwd`` through ``kda_chunk_fwd_noalloc``: the library takes its
    workspace from a static device array of ``NOALLOC_SCRATCH_BYTES`` (one per
    GPU) and allocates nothing.  This wrapper still allocates ``out`` and
    ``final_state`` with torch unless they are passed in.  Calls that overlap
    on one GPU race on that array.  Returns ``(out, final_state)``."""
    lib = load_library()
    if q.dim() != 4:
        raise ValueError("q must be [B, T, H, dk]")
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("kda.chunk_fwd_noalloc runs on a HIP device; tensors are on " + str(dev))
    dt = q.dtype
    code = _dtype_code(dt)
    chunk = _DEFAULT_CHUNK[code] if chunk is None else int(chunk)
    for name, t, shp in (("q", q, (B, T, H, dk)), ("k", k, (B, T, H, dk)),
                         ("g", g, (B, T, H, dk)), ("v", v, (B, T, H, dv)),
                         ("gate", gate, (B, T, H, dv)), ("beta", beta, (B, T, H))):
        _need(t, name, shp, dt, dev)
    if cu_seqlens is not None:
        if cu_seqlens.dtype != torch.int32 or cu_seqlens.dim() != 1:
            raise TypeError("cu_seqlens must be a 1-D int32 tensor")
        _need(cu_seqlens, "cu_seqlens", cu_seqlens.shape, torch.int32, dev)
        N = cu_seqlens.numel() - 1
    else:
        N = B
    if init_state is not None:
        _need(init_state, "init_state", (N, H, dk, dv), torch.float32, dev)
    if out is None:
        out = torch.empty((B, T, H, dv), dtype=dt, device=dev)
    else:
        _need(out, "out", (B, T, H, dv), dt, dev)
    if output_final_state:
        if final_state is None:
            final_state = torch.empty((N, H, dk, dv), dtype=torch.float32, device=dev)
        else:
            _need(final_state, "final_state", (N, H, dk, dv), torch.float32, dev)
    else:
        final_state = None
    st = lib.kda_chunk_fwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(gate),
                                   _ptr(init_state), _ptr(out), _ptr(final_state),
                                   _ptr(cu_seqlens), B, T, N, H, dk, dv, chunk, float(scale),
                                   code, _stream_ptr(dev))
    _check(st)
    return out, final_state


def chunk_fwd_snapshots(q, k, v, g, beta, gate, interval, init_state=None,
                        output_final_state=True, cu_seqlens=None, chunk=None, scale=1.0,
                        workspace=None, out=None, final_state=None, snapshots=None, prologue=0):
    """``chunk_fwd`` that also returns fp32 state snapshots every ``interval``
    tokens of each sequence (a multiple of the chunk length), as
    ``[snapshot_slots(...), H, dk, dv]``; ``snapshot_index`` maps slots to
    (sequence, token count).  Returns ``(out, final_state, snapshots)``."""
    return _chunk_call(q, k, v, g, beta, gate, init_state, output_final_state, cu_seqlens,
                       chunk, scale, workspace, out, final_state, interval, snapshots, prologue)


def decode_step(q, k, v, g, beta, gate, state, scale=1.0, out=None, prologue=0):
    """One recurrent KDA step on the GPU; ``state`` (fp32 ``[N, H, dk, dv]``)
    is updated in place.  q, k, g ``[N, H, dk]``; v, gate ``[N, H, dv]``;
    beta ``[N, H]``.  Returns the gated output ``[N, H, dv]``."""
    lib = load_library()
    if state.dim() != 4:
        raise ValueError("state must be [N, H, dk, dv]")
    N, H, dk, dv = state.shape
    dev = state.device
    if dev.type != "cuda":
        raise ValueError("kda.decode_step runs on a HIP device; state is on " + str(dev))
    _need(state, "state", (N, H, dk, dv), torch.float32, dev)
    dt = q.dtype
    code = _dtype_code(dt)
    for name, t, shp in (("q", q, (N, H, dk)), ("k", k, (N, H, dk)), ("g", g, (N, H, dk)),
                         ("v", v, (N, H, dv)), ("gate", gate, (N, H, dv)), ("beta", beta, (N, H))):
        _need(t, name, shp, dt, dev)
    if out is None:
        out = torch.empty((N, H, dv), dtype=dt, device=dev)
    else:
        _need(out, "out", (N, H, dv), dt, dev)
    if prologue:
        st = lib.kda_decode_step_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(gate),
                                    _ptr(state), _ptr(out), N, H, dk, dv, float(scale), code,
                                    int(prologue), _stream_ptr(dev))
    else:
        st = lib.kda_decode_step(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(gate),
                                 _ptr(state), _ptr(out), N, H, dk, dv, float(scale), code,
                                 _stream_ptr(dev))
    _check(st)
    return out


def decode_verify(q, k, v, g, beta, gate, state, scale=1.0, prologue=0, out=None, u=None):
    """Run K draft tokens per sequence from ``state`` (fp32 ``[N, H, dk, dv]``,
    not modified).  q, k, g ``[N, K, H, dk]``; v, gate ``[N, K, H, dv]``; beta
    ``[N, K, H]``.  Returns ``(out [N, K, H, dv], u [N, K, H, dv] fp32)``; pass
    ``u`` and the same k, g to ``decode_commit`` once the accepted prefix is
    known."""
    lib = load_library()
    if state.dim() != 4 or q.dim() != 4:
        raise ValueError("state must be [N, H, dk, dv] and q [N, K, H, dk]")
    N, H, dk, dv = state.shape
    dev = state.device
    if dev.type != "cuda":
        raise ValueError("kda.decode_verify runs on a HIP device; state is on " + str(dev))
    _need(state, "state", (N, H, dk, dv), torch.float32, dev)
    K = q.shape[1]
    dt = q.dtype
    code = _dtype_code(dt)
    for name, t, shp in (("q", q, (N, K, H, dk)), ("k", k, (N, K, H, dk)),
                         ("g", g, (N, K, H, dk)), ("v", v, (N, K, H, dv)),
                         ("gate", gate, (N, K, H, dv)), ("beta", beta, (N, K, H))):
        _need(t, name, shp, dt, dev)
    if out is None:
        out = torch.empty((N, K, H, dv), dtype=dt, device=dev)
    else:
        _need(out, "out", (N, K, H, dv), dt, dev)
    if u is None:
        u = torch.empty((N, K, H, dv), dtype=torch.float32, device=dev)
    else:
        _need(u, "u", (N, K, H, dv), torch.float32, dev)
    st = lib.kda_decode_verify(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(gate),
                               _ptr(state), _ptr(out), _ptr(u), N, K, H, dk, dv, float(scale),
                               code, int(prologue), _stream_ptr(dev))
    _check(st)
    return out, u


def decode_commit(k, g, u, accepted, state, prologue=0):
    """Advance ``state`` (in place) past the first ``accepted[n]`` verified
    tokens of each sequence (``accepted``: int32 ``[N]`` on the device), using
    the k, g and ``u`` of ``decode_verify``."""
    lib = load_library()
    N, H, dk, dv = state.shape
    dev = state.device
    if dev.type != "cuda":
        raise ValueError("kda.decode_commit runs on a HIP device; state is on " + str(dev))
    _need(state, "state", (N, H, dk, dv), torch.float32, dev)
    K = k.shape[1]
    dt = k.dtype
    code = _dtype_code(dt)
    _need(k, "k", (N, K, H, dk), dt, dev)
    _need(g, "g", (N, K, H, dk), dt, dev)
    _need(u, "u", (N, K, H, dv), torch.float32, dev)
    _need(accepted, "accepted", (N,), torch.int32, dev)
    st = lib.kda_decode_commit(_ptr(k), _ptr(g), _ptr(u), _ptr(accepted), _ptr(state), N, K, H,
                               dk, dv, code, int(prologue), _stream_ptr(dev))
    _check(st)


def chunk_bwd_supported(dtype: torch.dtype, dk: int, dv: int, chunk: int) -> bool:
    return bool(load_library().kda_chunk_bwd_supported(_dtype_code(dtype), dk, dv, chunk))


def chunk_bwd_workspace_bytes(B: int, T: int, N: int, H: int, dk: int, dv: int, chunk: int,
                              dtype: torch.dtype, varlen: bool) -> int:
    n = load_library().kda_chunk_bwd_workspace_bytes(B, T, N, H, dk, dv, chunk,
                                                     _dtype_code(dtype), int(varlen))
    if n == ctypes.c_size_t(-1).value:
        raise KdaError("unsupported or invalid sizes for kda_chunk_bwd")
    return int(n)


def chunk_bwd(q, k, v, g, beta, gate, grad_out, init_state=None, grad_final_state=None,
              cu_seqlens=None, chunk=None, scale=1.0, workspace=None, want_grad_init=True,
              grads=None, fwd_workspace=None):
    """Chunkwise KDA backward on the GPU: gradients of a loss with respect to
    every input of ``chunk_fwd`` (prepared inputs), given ``grad_out`` (shape
    and dtype of the forward's ``out``) and optionally ``grad_final_state``
    (fp32 ``[N, H, dk, dv]``).  Returns a dict with ``q, k, v, g, beta, gate``
    (the input dtype) and ``init_state`` (fp32, None unless ``want_grad_init``).
    ``grads``: an optional dict of preallocated outputs with those keys.
    ``fwd_workspace``: the workspace of a ``chunk_fwd(..., chunk_records=True)``
    call on the same inputs (bf16, no prologue), untouched since; its records
    are reused and consumed."""
    lib = load_library()
    if q.dim() != 4:
        raise ValueError("q must be [B, T, H, dk]")
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("kda.chunk_bwd runs on a HIP device; tensors are on " + str(dev))
    dt = q.dtype
    code = _dtype_code(dt)
    chunk = _DEFAULT_CHUNK[code] if chunk is None else int(chunk)
    for name, t, shp in (("q", q, (B, T, H, dk)), ("k", k, (B, T, H, dk)),
                         ("g", g, (B, T, H, dk)), ("v", v, (B, T, H, dv)),
                         ("gate", gate, (B, T, H, dv)), ("beta", beta, (B, T, H)),
                         ("grad_out", grad_out, (B, T, H, dv))):
        _need(t, name, shp, dt, dev)
    if cu_seqlens is not None:
        if cu_seqlens.dtype != torch.int32 or cu_seqlens.dim() != 1:
            raise TypeError("cu_seqlens must be a 1-D int32 tensor")
        _need(cu_seqlens, "cu_seqlens", cu_seqlens.shape, torch.int32, dev)
        if B != 1:
            raise ValueError("cu_seqlens requires B == 1")
        N = cu_seqlens.numel() - 1
    else:
        N = B
    if init_state is not None:
        _need(init_state, "init_state", (N, H, dk, dv), torch.float32, dev)
    if grad_final_state is not None:
        _need(grad_final_state, "grad_final_state", (N, H, dk, dv), torch.float32, dev)
    nbytes = chunk_bwd_workspace_bytes(B, T, N, H, dk, dv, chunk, dt, cu_seqlens is not None)
    if fwd_workspace is not None:
        if fwd_workspace.device != dev or fwd_workspace.dtype != torch.uint8:
            raise ValueError(f"fwd_workspace must be a uint8 tensor on {dev}")
        nbytes -= chunk_fwd_workspace_bytes(B, T, N, H, dk, dv, chunk, dt,
                                            cu_seqlens is not None, chunk_records=True)
    if workspace is None:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)
    elif workspace.device != dev or workspace.dtype != torch.uint8 or workspace.numel() < nbytes:
        raise ValueError(f"workspace must be a uint8 tensor of at least {nbytes} bytes on {dev}")
    if grads is None:
        grads = {name: torch.empty_like(t) for name, t in
                 (("q", q), ("k", k), ("v", v), ("g", g), ("beta", beta), ("gate", gate))}
        grads["init_state"] = (torch.empty((N, H, dk, dv), dtype=torch.float32, device=dev)
                               if want_grad_init else None)
    else:
        for name, t in (("q", q), ("k", k), ("v", v), ("g", g), ("beta", beta), ("gate", gate)):
            _need(grads[name], "grads['" + name + "']", t.shape, dt, dev)
        if grads.get("init_state") is not None:
            _need(grads["init_state"], "grads['init_state']", (N, H, dk, dv), torch.float32, dev)
    st = lib.kda_chunk_bwd_ex(
        _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(gate), _ptr(init_state),
        _ptr(grad_out), _ptr(grad_final_state), _ptr(grads["q"]), _ptr(grads["k"]),
        _ptr(grads["v"]), _ptr(grads["g"]), _ptr(grads["beta"]), _ptr(grads["gate"]),
        _ptr(grads["init_state"]), _ptr(cu_seqlens), B, T, N, H, dk, dv, chunk, float(scale),
        code, _ptr(fwd_workspace), 0 if fwd_workspace is None else fwd_workspace.numel(),
        _ptr(workspace), workspace.numel(), _stream_ptr(dev))
    _check(st)
    return grads
