"""GPU parity of speculative verification and commit.

decode_verify(K tokens) must return, for every token, what successive
decode_step calls return (bit for bit, and against the oracle within the
decode tolerance) and leave the state unchanged; decode_commit(accepted)
must leave the state equal to accepted[n] successive decode steps (bit for
bit, and against the oracle's state)."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import kimi_delta_attention_chunkwise_amd as kda
import oracle
from oracle import prologue as P
from test_gpu_parity import TOL_BF16_OUT, dev, np32, rel, say  # noqa: F401

pytestmark = pytest.mark.gpu

KEYS = ("q", "k", "v", "g", "beta", "z")


def draft_inputs(dtype, N, K, H, d, seed, raw):
    gen = torch.Generator().manual_seed(seed)
    n = lambda *s: torch.randn(*s, generator=gen)
    q, k = n(N, K, H, d), n(N, K, H, d)
    beta, g = n(N, K, H), n(N, K, H, d)
    if not raw:
        q = q / q.norm(dim=-1, keepdim=True)
        k = k / k.norm(dim=-1, keepdim=True)
        beta = torch.sigmoid(beta)
        g = torch.clamp(-torch.nn.functional.softplus(g), min=-5.0)
    d_ = {"q": q, "k": k, "v": n(N, K, H, d), "g": g, "beta": beta, "z": n(N, K, H, d)}
    return {key: val.to(dtype) for key, val in d_.items()}


# K = 5 and 9 leave a ragged last group of the four-token staging; K = 1 and 8 do not
@pytest.mark.parametrize("dtype,d,pro,K", [(torch.bfloat16, 128, 0, 5), (torch.float32, 16, 0, 5),
                                           (torch.bfloat16, 128, 7, 5), (torch.float32, 128, 0, 5),
                                           (torch.bfloat16, 128, 0, 1), (torch.bfloat16, 128, 7, 8),
                                           (torch.float32, 16, 7, 9)])
def test_verify_and_commit(dev, dtype, d, pro, K):
    N, H = 6, 3
    x = draft_inputs(dtype, N, K, H, d, 80 + d + pro + 100 * K, raw=bool(pro))
    xd = {key: val.to(dev) for key, val in x.items()}
    gen = torch.Generator().manual_seed(81)
    st0 = (torch.randn(N, H, d, d, generator=gen) * 0.05).to(dev)
    state = st0.clone()
    out, u = kda.decode_verify(xd["q"], xd["k"], xd["v"], xd["g"], xd["beta"], xd["z"], state,
                               prologue=pro)
    torch.cuda.synchronize()
    assert torch.equal(state, st0), "verification changed the state"

    # successive decode steps on the GPU: states after 0 .. K tokens, outputs
    seq = st0.clone()
    states = [seq.clone()]
    outs = []
    for t in range(K):
        tok = {key: xd[key][:, t].contiguous() for key in KEYS}
        outs.append(kda.decode_step(tok["q"], tok["k"], tok["v"], tok["g"], tok["beta"],
                                    tok["z"], seq, prologue=pro))
        states.append(seq.clone())
    torch.cuda.synchronize()
    assert torch.equal(out, torch.stack(outs, dim=1)), "verify outputs differ from decode steps"

    # the oracle over the same K tokens
    ref = st0.double().cpu().numpy().copy()
    ref_states = [ref.copy()]
    worst = 0.0
    for t in range(K):
        tok = {key: np32(x[key][:, t]) for key in KEYS}
        q, k, beta, g = P.apply(tok["q"], tok["k"], tok["beta"], tok["g"], pro)
        ry = oracle.decode_step(q, k, tok["v"].astype(np.float64), g, beta,
                                tok["z"].astype(np.float64), ref)
        worst = max(worst, rel(np32(out[:, t]), ry))
        ref_states.append(ref.copy())
    tol_out = TOL_BF16_OUT if dtype == torch.bfloat16 else 1e-5
    say(f"verify {dtype} d={d} prologue={pro} K={K}: worst out rel err {worst:.3e}")
    assert worst <= tol_out

    # commit: accepted prefix lengths 0 .. K (and out-of-range values clamp)
    acc = torch.tensor([0, 1, 2, K, 3, K + 7], dtype=torch.int32)
    committed = st0.clone()
    kda.decode_commit(xd["k"], xd["g"], u, acc.to(dev), committed, prologue=pro)
    torch.cuda.synchronize()
    worst_s = 0.0
    for n_ in range(N):
        a = min(max(int(acc[n_]), 0), K)
        assert torch.equal(committed[n_], states[a][n_]), f"sequence {n_}: commit of {a} tokens"
        worst_s = max(worst_s, rel(np32(committed[n_]), ref_states[a][n_]))
    say(f"commit {dtype} d={d} prologue={pro} K={K}: worst state rel err {worst_s:.3e}")
    assert worst_s <= 1e-4
