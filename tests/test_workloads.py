"""The seeded input generators: determinism, shapes and the stated ranges."""
import torch

import workloads as W


def test_prefill_inputs_are_deterministic_and_in_range():
    w = W.WORKLOADS["tiny_f32"]
    a = W.prefill_inputs(w, seed=3)
    b = W.prefill_inputs(w, seed=3)
    for key in ("q", "k", "v", "g", "beta", "z"):
        assert torch.equal(a[key], b[key])
    assert a["q"].shape == (1, 64, 2, 16) and a["q"].dtype == torch.float32
    assert a["beta"].shape == (1, 64, 2)
    assert float(a["g"].min()) >= -5.0 and float(a["g"].max()) < 0.0
    assert float(a["beta"].min()) > 0.0 and float(a["beta"].max()) < 1.0
    n = torch.linalg.vector_norm(a["k"].double(), dim=-1)
    assert torch.allclose(n, torch.ones_like(n), atol=1e-6)
    c = W.prefill_inputs(w, seed=4)
    assert not torch.equal(a["q"], c["q"])


def test_varlen_lengths_and_packing():
    w = W.WORKLOADS["varlen_4seq_h32"]
    lens = W.varlen_lengths(w, seed=0)
    assert len(lens) == 4 and all(1024 <= x <= 32768 for x in lens)
    assert lens == W.varlen_lengths(w, seed=0)
    small = W.prefill_inputs(w, seed=0, lengths=[5, 0, 17])
    assert small["cu_seqlens"].tolist() == [0, 5, 5, 22]
    assert small["q"].shape == (1, 22, 32, 128) and small["q"].dtype == torch.bfloat16
    assert small["init_state"].shape == (3, 32, 128, 128)
    assert abs(float(small["init_state"].std()) - 0.02) < 0.002


def test_pinned_channels_quarter_of_dk():
    w = W.WORKLOADS["long_t1m_h16"]
    m = W.pinned_channels(w, seed=0)
    assert m.shape == (16, 128) and m.sum(dim=1).tolist() == [32] * 16
    x = W.prefill_inputs(w, seed=0, T=40)
    g = x["g"][0].float()                       # [T, H, dk]
    assert torch.all(g[:, m] == -5.0)
    assert torch.all(g[:, ~m] >= -5.0)


def test_decode_inputs_shapes():
    w = W.WORKLOADS["decode_n256_h32"]
    d = W.decode_inputs(w, step=0, N=4)
    assert d["q"].shape == (4, 32, 128) and d["beta"].shape == (4, 32)
    assert not torch.equal(d["q"], W.decode_inputs(w, step=1, N=4)["q"])
