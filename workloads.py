"""Seeded synthetic KDA workloads: shapes and input generators.

This module holds no KDA arithmetic.  It only draws inputs with the
distributions the five workloads name and casts them to the workload dtype,
so both the HIP path and the CPU oracle can be fed the very same tensors.

Input recipe (every workload):
  q, k  ~ N(0, 1), then L2-normalised over dk per (token, head), in float32
  v     ~ N(0, 1)
  beta  = sigmoid(x), x ~ N(0, 1)           (a value in (0, 1) per token-head)
  g     = max(-5, -softplus(x)), x ~ N(0, 1) (natural-log decay per key channel;
                                             the lower bound -5 is the log-decay
                                             floor of the chunked kernel)
  z     ~ N(0, 1)                            (gate logit; the gate is sigmoid(z))
  init  ~ N(0, 0.02^2), float32, only where a workload asks for one
Draws are float32 from a ``torch.Generator`` seeded with (workload id, seed)
on the requested device, then rounded to nearest-even into the dtype.
Values on CPU and GPU generators differ (different streams); a test always
feeds both sides the same tensors.

Workloads (dk = dv = 128 unless noted; scale = 1):
  tiny_f32          fp32, B=1, H=2, T=64, dk=dv=16, chunk 16, zero init
  prefill_t4096_h8  bf16, B=1, H=8, T=4096, chunk 64 (4 x 16-token subtiles)
  varlen_4seq_h32   bf16, 4 sequences, lengths uniform on [1024, 32768]
                    (integers, inclusive) packed with cu_seqlens, H=32,
                    init ~ N(0, 0.02^2) per sequence
  long_t1m_h16      bf16, B=1, H=16, T=1,048,576; for every head a seeded
                    random quarter of the key channels has g = -5 at every
                    token; the state after T/2 seeds the second half
  decode_n256_h32   bf16 q/k/v/g/beta/z, fp32 state [256, 32, 128, 128],
                    one token per step, 128 steps, zero init
"""
from __future__ import annotations

import dataclasses

import torch

G_MIN = -5.0


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    wid: int
    dtype: str            # "f32" or "bf16": dtype of q, k, v, g, beta, z and out
    H: int
    dk: int
    dv: int
    B: int = 1
    T: int = 0            # per-sequence length (fixed-length workloads)
    chunk: int = 64
    n_seq: int = 0        # varlen: number of packed sequences
    len_lo: int = 0
    len_hi: int = 0
    init_std: float = 0.0  # 0 => zero initial state
    pinned_frac: float = 0.0
    N: int = 0            # decode: concurrent sequences
    steps: int = 0        # decode: steps

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == "f32" else torch.bfloat16


WORKLOADS = {
    w.name: w
    for w in [
        Workload("tiny_f32", 0, "f32", H=2, dk=16, dv=16, B=1, T=64, chunk=16),
        Workload("prefill_t4096_h8", 1, "bf16", H=8, dk=128, dv=128, B=1, T=4096, chunk=64),
        Workload("varlen_4seq_h32", 2, "bf16", H=32, dk=128, dv=128, n_seq=4, len_lo=1024,
                 len_hi=32768, init_std=0.02, chunk=64),
        Workload("long_t1m_h16", 3, "bf16", H=16, dk=128, dv=128, B=1, T=1 << 20, chunk=64,
                 pinned_frac=0.25),
        Workload("decode_n256_h32", 4, "bf16", H=32, dk=128, dv=128, N=256, steps=128),
    ]
}


def _gen(wid: int, seed: int, stream: int, device) -> torch.Generator:
    gen = torch.Generator(device=device)
    gen.manual_seed((wid * 1_000_003 + seed * 7919 + stream * 104_729) & 0x7FFF_FFFF_FFFF_FFFF)
    return gen


def varlen_lengths(w: Workload, seed: int = 0) -> list[int]:
    """Sequence lengths for a varlen workload (seeded, CPU generator)."""
    gen = _gen(w.wid, seed, 99, "cpu")
    x = torch.randint(w.len_lo, w.len_hi + 1, (w.n_seq,), generator=gen)
    return [int(v) for v in x]


def draw_tokens(shape_tok, H, dk, dv, dtype, gen, device, pinned_mask=None):
    """q, k, v, g, beta, z for ``shape_tok`` leading token dims (e.g. (B, T)).

    ``pinned_mask``: optional bool [H, dk]; True channels get g = -5 everywhere.
    """
    shp = tuple(shape_tok)

    def normal(*s):
        return torch.randn(*s, generator=gen, device=device, dtype=torch.float32)

    def unit(x):
        return x / torch.linalg.vector_norm(x, dim=-1, keepdim=True).clamp_min(1e-30)

    q = unit(normal(*shp, H, dk)).to(dtype)
    k = unit(normal(*shp, H, dk)).to(dtype)
    v = normal(*shp, H, dv).to(dtype)
    g = torch.clamp(-torch.nn.functional.softplus(normal(*shp, H, dk)), min=G_MIN)
    if pinned_mask is not None:
        g = torch.where(pinned_mask.to(device), torch.full_like(g, G_MIN), g)
    g = g.to(dtype)
    beta = torch.sigmoid(normal(*shp, H)).to(dtype)
    z = normal(*shp, H, dv).to(dtype)
    return dict(q=q, k=k, v=v, g=g, beta=beta, z=z)


def pinned_channels(w: Workload, seed: int = 0) -> torch.Tensor | None:
    """Bool [H, dk]: a seeded random set of round(pinned_frac * dk) channels per head."""
    if w.pinned_frac <= 0:
        return None
    gen = _gen(w.wid, seed, 77, "cpu")
    n = int(round(w.pinned_frac * w.dk))
    mask = torch.zeros(w.H, w.dk, dtype=torch.bool)
    for h in range(w.H):
        mask[h, torch.randperm(w.dk, generator=gen)[:n]] = True
    return mask


def prefill_inputs(w: Workload, device="cpu", seed: int = 0, T: int | None = None,
                   lengths: list[int] | None = None):
    """Inputs for a prefill workload, laid out [B, T, H, d] (varlen: B = 1).

    ``T`` overrides the fixed length (for smaller test cases of the same shape);
    ``lengths`` overrides the varlen lengths.  Returns a dict with q, k, v, g,
    beta, z, init_state (or None), cu_seqlens (int32, or None) and N.
    """
    gen = _gen(w.wid, seed, 1, device)
    if w.n_seq:
        lens = lengths if lengths is not None else varlen_lengths(w, seed)
        total = int(sum(lens))
        tok = (1, total)
        cu = torch.zeros(len(lens) + 1, dtype=torch.int32)
        cu[1:] = torch.cumsum(torch.tensor(lens, dtype=torch.int64), 0).to(torch.int32)
        N = len(lens)
    else:
        tok = (w.B, T if T is not None else w.T)
        cu = None
        N = w.B
    d = draw_tokens(tok, w.H, w.dk, w.dv, w.torch_dtype, gen, device, pinned_channels(w, seed))
    init = None
    if w.init_std > 0:
        init = (torch.randn(N, w.H, w.dk, w.dv, generator=gen, device=device) * w.init_std)
    d.update(init_state=init, cu_seqlens=None if cu is None else cu.to(device), N=N)
    return d


def decode_inputs(w: Workload, step: int, device="cpu", seed: int = 0, N: int | None = None):
    """One decode step's inputs: q, k, g [N, H, dk]; v, z [N, H, dv]; beta [N, H]."""
    gen = _gen(w.wid, seed, 1000 + step, device)
    return draw_tokens((N if N is not None else w.N,), w.H, w.dk, w.dv, w.torch_dtype, gen, device)


def decode_init_state(w: Workload, device="cpu", seed: int = 0, N: int | None = None,
                      std: float = 0.0):
    n = N if N is not None else w.N
    if std <= 0:
        return torch.zeros(n, w.H, w.dk, w.dv, device=device, dtype=torch.float32)
    gen = _gen(w.wid, seed, 5, device)
    return torch.randn(n, w.H, w.dk, w.dv, generator=gen, device=device) * std
