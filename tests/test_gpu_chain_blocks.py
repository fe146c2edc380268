"""GPU: chain workgroups that own several value blocks.

When the chain's one-block workgroups (N * H * 8) outnumber the CUs, the chain
runs with 4 (or 2) value blocks per workgroup, which stream the L operand once
for all of them.  Every value block goes through the same arithmetic as with
one block per workgroup, so the results must be bitwise those of per-head
calls (H = 1, which always runs one block per workgroup): outputs and final
states of the forward, and every gradient of the backward.
"""
from __future__ import annotations

import pytest
import torch

import kimi_delta_attention_chunkwise_amd as kda

from test_gpu_parity import small_inputs, to

pytestmark = pytest.mark.gpu
KEYS = ("q", "k", "v", "g", "beta", "z")


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no HIP device")
    kda.load_library()
    return torch.device("cuda:0")


def say(msg):
    print(f"[gpu-chain-blocks] {msg}", flush=True)


def head(xd, h):
    d = {k: xd[k][:, :, h:h + 1].contiguous() for k in KEYS}
    d["init_state"] = None if xd.get("init_state") is None else \
        xd["init_state"][:, h:h + 1].contiguous()
    d["cu_seqlens"] = xd.get("cu_seqlens")
    return d


CASES = {
    # name: (B, T, H, lengths); units = sequences x heads
    "varlen_64_units": (1, 0, 32, [300, 129]),            # 2 blocks per workgroup
    "varlen_128_units": (1, 0, 32, [200, 1, 64, 77]),     # 4 blocks per workgroup
    "batch_160_units": (5, 130, 32, None),                # 4 blocks per workgroup
}


@pytest.mark.parametrize("case", list(CASES))
def test_multi_block_chain_equals_per_head_calls(dev, case):
    B, T, H, lengths = CASES[case]
    say(f"{case}: B={B} T={T} H={H} lengths={lengths}")
    xd = to(small_inputs(torch.bfloat16, B, T, H, 128, 128, 90, lengths=lengths, init_std=0.02),
            dev)
    out, fin = kda.chunk_fwd(*[xd[k] for k in KEYS], init_state=xd["init_state"],
                             cu_seqlens=xd["cu_seqlens"])
    torch.cuda.synchronize()
    for h in range(H):
        d = head(xd, h)
        o, f = kda.chunk_fwd(*[d[k] for k in KEYS], init_state=d["init_state"],
                             cu_seqlens=d["cu_seqlens"])
        torch.cuda.synchronize()
        assert torch.equal(out[:, :, h:h + 1], o), f"{case}: head {h} output differs"
        assert torch.equal(fin[:, h:h + 1], f), f"{case}: head {h} final state differs"


def test_multi_block_chain_backward_equals_per_head_calls(dev):
    lengths = [200, 1, 64, 77]
    H = 32
    say(f"backward, lengths={lengths}, H={H} (4 blocks per chain workgroup)")
    xd = to(small_inputs(torch.bfloat16, 1, 0, H, 128, 128, 91, lengths=lengths, init_std=0.02),
            dev)
    gen = torch.Generator().manual_seed(92)
    dy = (torch.randn(xd["q"].shape[:3] + (128,), generator=gen)).to(torch.bfloat16).to(dev)
    dfin = (torch.randn(len(lengths), H, 128, 128, generator=gen) * 0.05).to(dev)
    gr = kda.chunk_bwd(*[xd[k] for k in KEYS], dy, init_state=xd["init_state"],
                       grad_final_state=dfin, cu_seqlens=xd["cu_seqlens"])
    torch.cuda.synchronize()
    for h in range(H):
        d = head(xd, h)
        g1 = kda.chunk_bwd(*[d[k] for k in KEYS], dy[:, :, h:h + 1].contiguous(),
                           init_state=d["init_state"],
                           grad_final_state=dfin[:, h:h + 1].contiguous(),
                           cu_seqlens=d["cu_seqlens"])
        torch.cuda.synchronize()
        for key in ("q", "k", "v", "g", "beta", "gate"):
            assert torch.equal(gr[key][:, :, h:h + 1], g1[key]), f"head {h}: d{key} differs"
        assert torch.equal(gr["init_state"][:, h:h + 1], g1["init_state"]), \
            f"head {h}: dS0 differs"
