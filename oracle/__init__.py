"""CPU oracle for Kimi Delta Attention (KDA) -- test infrastructure only.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  It shares no code with the HIP path in
``kimi_delta_attention_chunkwise_amd``; neither imports the other.

Contents
  * ``forward`` / ``decode_step``: the plain token-by-token recurrence in fp64,
    in C (``kda_oracle.c``, OpenMP over (sequence, head) units), loaded with
    ctypes.  This is the oracle the GPU path is compared against.
  * ``forward_compare``: the same recurrence compared on the fly with an
    output computed elsewhere (per (sequence, head) maximum errors), for
    inputs too long to hold a float64 output; bfloat16 inputs are widened
    exactly.
  * ``backward``: reverse-mode gradients of ``forward`` in fp64, token by
    token (same C file).
  * ``oracle.chunkwise``: a second fp64 implementation in NumPy that follows
    the chunkwise-parallel form (state passed between chunks, matrices inside a
    chunk).  Used to check that the chunkwise form equals the recurrence.
  * ``oracle.exact``: exact rational arithmetic (``fractions``) on tiny inputs,
    in the dense matrix form of the update.  Pins the C loop.

Sources: "Kimi K3 second-pass study ledger" (llm-atlas K3_RESEARCH.md),
section 1, rows Q04, Q05, Q07, Q08; "Kimi K3 plain-language guide", section 5.1.
Parity unpinned against the report's own KDA equation, which the pages cite
but do not print.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kda_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile kda_oracle.c into liboracle.so with gcc (OpenMP, -O3)."""
    if not force and os.path.exists(_LIB_PATH):
        return _LIB_PATH
    tmp = _LIB_PATH + ".tmp"
    cmd = ["gcc", "-std=c99", "-O3", "-fopenmp", "-fPIC", "-shared", _SRC, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    # KDA_ORACLE_LIB lets the mutation test point the pins at a deliberately
    # broken copy of the oracle; normal runs never set it.
    path = os.environ.get("KDA_ORACLE_LIB", "")
    if not path:
        path = _LIB_PATH
        if not os.path.exists(path):
            build()
    lib = ctypes.CDLL(path)
    vp, dp, i64p = ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p
    i64, f64, cint = ctypes.c_int64, ctypes.c_double, ctypes.c_int
    lib.kda_oracle_forward.argtypes = [vp, vp, vp, vp, vp, vp, cint, dp, dp, dp, i64p,
                                       i64, i64, i64, i64, f64, cint]
    lib.kda_oracle_forward.restype = cint
    lib.kda_oracle_decode_step.argtypes = [vp, vp, vp, vp, vp, vp, cint, dp, dp,
                                           i64, i64, i64, i64, f64, cint]
    lib.kda_oracle_decode_step.restype = cint
    lib.kda_oracle_backward.argtypes = [vp, vp, vp, vp, vp, vp, cint, dp, dp, dp, i64p,
                                        i64, i64, i64, i64, f64, cint,
                                        dp, dp, dp, dp, dp, dp, dp]
    lib.kda_oracle_backward.restype = cint
    lib.kda_oracle_forward_compare.argtypes = [vp, vp, vp, vp, vp, vp, cint, dp, vp, cint, i64p,
                                               i64, i64, i64, i64, f64, cint, dp, dp, dp]
    lib.kda_oracle_forward_compare.restype = cint
    lib.kda_oracle_max_threads.argtypes = []
    lib.kda_oracle_max_threads.restype = cint
    _lib = lib
    return lib


def max_threads() -> int:
    return int(_load().kda_oracle_max_threads())


def _as_input(x, in_f32):
    x = np.asarray(x)
    want = np.float32 if in_f32 else np.float64
    return np.ascontiguousarray(x, dtype=want)


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p) if a is not None else None


def forward(q, k, v, g, beta, z, init_state=None, cu_seqlens=None, scale=1.0,
            output_final_state=True, n_threads=None):
    """Token-by-token KDA forward in fp64.

    Shapes: q, k, g ``[B, T, H, dk]`` (or ``[T, H, dk]``), v, z ``[B, T, H, dv]``,
    beta ``[B, T, H]``.  With ``cu_seqlens`` (length N + 1) the leading batch
    dimension must be 1 (or absent) and the sequences are packed along T.
    ``init_state``: ``[N, H, dk, dv]`` or None (zeros).
    Inputs that are float32 are widened exactly; anything else is converted to
    float64 first.  Returns ``(out[B, T, H, dv] float64, final[N, H, dk, dv])``.
    """
    q = np.asarray(q)
    batched = q.ndim == 4
    if batched:
        B, T, H, dk = q.shape
    else:
        B = 1
        T, H, dk = q.shape
    dv = np.asarray(v).shape[-1]
    in_f32 = all(np.asarray(x).dtype == np.float32 for x in (q, k, v, g, beta, z))
    flat = lambda x, d: _as_input(np.asarray(x).reshape(B * T, H, d) if d else
                                  np.asarray(x).reshape(B * T, H), in_f32)
    qf, kf, gf = flat(q, dk), flat(k, dk), flat(g, dk)
    vf, zf = flat(v, dv), flat(z, dv)
    bf = flat(beta, 0)
    if cu_seqlens is None:
        cu = np.arange(B + 1, dtype=np.int64) * T
    else:
        if B != 1:
            raise ValueError("cu_seqlens needs a batch dimension of 1")
        cu = np.ascontiguousarray(np.asarray(cu_seqlens), dtype=np.int64)
        if cu[0] != 0 or cu[-1] != T or np.any(np.diff(cu) < 0):
            raise ValueError("cu_seqlens must start at 0, end at T and be non-decreasing")
    N = len(cu) - 1
    init = None
    if init_state is not None:
        init = np.ascontiguousarray(np.asarray(init_state), dtype=np.float64)
        if init.shape != (N, H, dk, dv):
            raise ValueError(f"init_state shape {init.shape} != {(N, H, dk, dv)}")
    out = np.empty((B * T, H, dv), dtype=np.float64)
    final = np.empty((N, H, dk, dv), dtype=np.float64) if output_final_state else None
    nt = n_threads if n_threads else max_threads()
    rc = _load().kda_oracle_forward(_ptr(qf), _ptr(kf), _ptr(vf), _ptr(gf), _ptr(bf), _ptr(zf),
                                    int(in_f32), _ptr(init), _ptr(out), _ptr(final), _ptr(cu),
                                    N, H, dk, dv, float(scale), int(nt))
    if rc != 0:
        raise RuntimeError(f"kda_oracle_forward failed with {rc}")
    out = out.reshape(B, T, H, dv) if batched else out.reshape(T, H, dv)
    return out, final


def forward_compare(q, k, v, g, beta, z, x, init_state=None, cu_seqlens=None, scale=1.0,
                    bf16=False, n_threads=None):
    """``forward`` compared on the fly with an output ``x`` computed elsewhere.

    Needs no float64 output array, so it serves inputs too long to hold one
    (a million tokens x 16 heads).  Inputs are float32 arrays, or with
    ``bf16=True`` uint16 arrays holding bfloat16 bit patterns (widened exactly);
    ``x`` is float32 or, with ``bf16=True``, bfloat16 bits, laid out like the
    output.  Shapes as in ``forward``.  Returns ``(err, ref, final)``: per
    (sequence, head) ``err[n, h] = max |x - y|`` and ``ref[n, h] = max |y|`` over
    that sequence's tokens and value channels (``y`` = the recurrence's output),
    and the final state ``[N, H, dk, dv]`` float64."""
    q = np.asarray(q)
    if q.ndim == 4:
        B, T, H, dk = q.shape
    else:
        B = 1
        T, H, dk = q.shape
    dv = np.asarray(v).shape[-1]
    want = np.uint16 if bf16 else np.float32
    arrs = [np.asarray(a) for a in (q, k, v, g, beta, z, x)]
    for a in arrs:
        if a.dtype != want or not a.flags["C_CONTIGUOUS"]:
            raise TypeError(f"forward_compare wants C-contiguous {np.dtype(want).name} arrays")
    if arrs[6].size != B * T * H * dv:
        raise ValueError("x must have the output's size")
    if cu_seqlens is None:
        cu = np.arange(B + 1, dtype=np.int64) * T
    else:
        if B != 1:
            raise ValueError("cu_seqlens needs a batch dimension of 1")
        cu = np.ascontiguousarray(np.asarray(cu_seqlens), dtype=np.int64)
        if cu[0] != 0 or cu[-1] != T or np.any(np.diff(cu) < 0):
            raise ValueError("cu_seqlens must start at 0, end at T and be non-decreasing")
    N = len(cu) - 1
    init = None
    if init_state is not None:
        init = np.ascontiguousarray(np.asarray(init_state), dtype=np.float64)
        if init.shape != (N, H, dk, dv):
            raise ValueError(f"init_state shape {init.shape} != {(N, H, dk, dv)}")
    err = np.empty((N, H), dtype=np.float64)
    ref = np.empty((N, H), dtype=np.float64)
    final = np.empty((N, H, dk, dv), dtype=np.float64)
    code = 2 if bf16 else 1
    nt = n_threads if n_threads else max_threads()
    rc = _load().kda_oracle_forward_compare(*(_ptr(a) for a in arrs[:6]), code, _ptr(init),
                                            _ptr(arrs[6]), code, _ptr(cu), N, H, dk, dv,
                                            float(scale), int(nt), _ptr(err), _ptr(ref),
                                            _ptr(final))
    if rc != 0:
        raise RuntimeError(f"kda_oracle_forward_compare failed with {rc}")
    return err, ref, final


def backward(q, k, v, g, beta, z, dout, init_state=None, dfinal=None, cu_seqlens=None,
             scale=1.0, n_threads=None):
    """Gradients of sum(dout * out) + sum(dfinal * final_state) for ``forward``.

    Same shapes and conventions as ``forward``; ``dout`` like ``out``, ``dfinal``
    like the final state (None = zero).  Returns a dict of float64 arrays:
    dq, dk, dv, dg, dbeta, dz (input shapes) and dinit ``[N, H, dk, dv]``."""
    q = np.asarray(q)
    batched = q.ndim == 4
    if batched:
        B, T, H, dk = q.shape
    else:
        B = 1
        T, H, dk = q.shape
    dv = np.asarray(v).shape[-1]
    in_f32 = all(np.asarray(x).dtype == np.float32 for x in (q, k, v, g, beta, z))
    flat = lambda x, d: _as_input(np.asarray(x).reshape(B * T, H, d) if d else
                                  np.asarray(x).reshape(B * T, H), in_f32)
    qf, kf, gf = flat(q, dk), flat(k, dk), flat(g, dk)
    vf, zf = flat(v, dv), flat(z, dv)
    bf = flat(beta, 0)
    if cu_seqlens is None:
        cu = np.arange(B + 1, dtype=np.int64) * T
    else:
        if B != 1:
            raise ValueError("cu_seqlens needs a batch dimension of 1")
        cu = np.ascontiguousarray(np.asarray(cu_seqlens), dtype=np.int64)
        if cu[0] != 0 or cu[-1] != T or np.any(np.diff(cu) < 0):
            raise ValueError("cu_seqlens must start at 0, end at T and be non-decreasing")
    N = len(cu) - 1
    init = None
    if init_state is not None:
        init = np.ascontiguousarray(np.asarray(init_state), dtype=np.float64)
        if init.shape != (N, H, dk, dv):
            raise ValueError(f"init_state shape {init.shape} != {(N, H, dk, dv)}")
    do = np.ascontiguousarray(np.asarray(dout, dtype=np.float64).reshape(B * T, H, dv))
    dfin = None
    if dfinal is not None:
        dfin = np.ascontiguousarray(np.asarray(dfinal), dtype=np.float64)
        if dfin.shape != (N, H, dk, dv):
            raise ValueError(f"dfinal shape {dfin.shape} != {(N, H, dk, dv)}")
    res = {"dq": np.empty((B * T, H, dk)), "dk": np.empty((B * T, H, dk)),
           "dv": np.empty((B * T, H, dv)), "dg": np.empty((B * T, H, dk)),
           "dbeta": np.empty((B * T, H)), "dz": np.empty((B * T, H, dv)),
           "dinit": np.empty((N, H, dk, dv))}
    nt = n_threads if n_threads else max_threads()
    rc = _load().kda_oracle_backward(
        _ptr(qf), _ptr(kf), _ptr(vf), _ptr(gf), _ptr(bf), _ptr(zf), int(in_f32), _ptr(init),
        _ptr(do), _ptr(dfin), _ptr(cu), N, H, dk, dv, float(scale), int(nt), _ptr(res["dq"]),
        _ptr(res["dk"]), _ptr(res["dv"]), _ptr(res["dg"]), _ptr(res["dbeta"]), _ptr(res["dz"]),
        _ptr(res["dinit"]))
    if rc != 0:
        raise RuntimeError(f"kda_oracle_backward failed with {rc}")
    shape_k = (B, T, H, dk) if batched else (T, H, dk)
    shape_v = (B, T, H, dv) if batched else (T, H, dv)
    shape_b = (B, T, H) if batched else (T, H)
    for key in ("dq", "dk", "dg"):
        res[key] = res[key].reshape(shape_k)
    for key in ("dv", "dz"):
        res[key] = res[key].reshape(shape_v)
    res["dbeta"] = res["dbeta"].reshape(shape_b)
    return res


def decode_step(q, k, v, g, beta, z, state, scale=1.0, n_threads=None):
    """One recurrent step on ``state`` ``[N, H, dk, dv]`` (float64, updated in
    place).  q, k, g ``[N, H, dk]``; v, z ``[N, H, dv]``; beta ``[N, H]``.
    Returns the gated output ``[N, H, dv]`` float64."""
    if not (isinstance(state, np.ndarray) and state.dtype == np.float64
            and state.flags["C_CONTIGUOUS"]):
        raise TypeError("state must be a C-contiguous float64 ndarray (updated in place)")
    N, H, dk, dv = state.shape
    in_f32 = all(np.asarray(x).dtype == np.float32 for x in (q, k, v, g, beta, z))
    qf, kf, gf = (_as_input(x, in_f32).reshape(N, H, dk) for x in (q, k, g))
    vf, zf = (_as_input(x, in_f32).reshape(N, H, dv) for x in (v, z))
    bf = _as_input(beta, in_f32).reshape(N, H)
    out = np.empty((N, H, dv), dtype=np.float64)
    nt = n_threads if n_threads else max_threads()
    rc = _load().kda_oracle_decode_step(_ptr(qf), _ptr(kf), _ptr(vf), _ptr(gf), _ptr(bf),
                                        _ptr(zf), int(in_f32), _ptr(state), _ptr(out),
                                        N, H, dk, dv, float(scale), int(nt))
    if rc != 0:
        raise RuntimeError(f"kda_oracle_decode_step failed with {rc}")
    return out
