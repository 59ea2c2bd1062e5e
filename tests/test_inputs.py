"""Seeded input generators: determinism, slice regeneration, recipes (CPU)."""
import numpy as np
import torch

from linear_attention_sequence_chunk_amd import inputs


def test_deterministic_and_sliceable():
    w = inputs.WORKLOADS["tiny"].with_(T=5000)   # spans two 4096-token blocks
    a = inputs.make_prefill(w)
    b = inputs.make_prefill(w)
    for key in ("q", "k", "v", "g", "beta"):
        assert torch.equal(a[key], b[key])
    part = inputs.make_prefill(w, t0=4000, t1=4200, heads=[1])
    for key in ("q", "k", "v", "g", "beta"):
        assert torch.equal(part[key], a[key][:, 4000:4200, [1]])


def test_recipes_tiny():
    w = inputs.WORKLOADS["tiny"]
    d = inputs.make_prefill(w)
    n = torch.linalg.vector_norm(d["q"].double(), dim=-1)
    assert torch.allclose(n, torch.ones_like(n), atol=1e-6)
    g = d["g"].double()
    assert (g < 0).all()
    alpha = g.exp()
    assert 0.12 < alpha.mean().item() < 0.19            # about 0.155
    assert ((d["beta"] > 0) & (d["beta"] < 1)).all()
    assert d["S0"] is None


def test_recipes_long_gates():
    w = inputs.WORKLOADS["long"].with_(T=512)
    d = inputs.make_prefill(w)
    alpha = d["g"].double().exp()
    fast = inputs._fast_channels(w)                       # [B,H,dk]
    assert 0.05 < fast.mean() < 0.15
    f = torch.from_numpy(fast)[:, None].expand_as(alpha)
    assert ((alpha[f] > 0.449) & (alpha[f] < 0.551)).all()
    assert ((alpha[~f] > 0.949) & (alpha[~f] < 0.9991)).all()
    assert d["S0"].shape == (1, 32, 128, 128) and abs(d["S0"].std().item() - 0.01) < 1e-3
    assert d["q"].dtype == torch.bfloat16


def test_address_keys_recur():
    w = inputs.WORKLOADS["1m"].with_(T=8192, H=2)
    d = inputs.make_prefill(w, gates="none")
    k = d["k"].double()
    # token p and p + 4096 (p < 64) share an address: high cosine; other tokens do not
    c_addr = (k[0, 10] * k[0, 4096 + 10]).sum(-1)
    c_free = (k[0, 100] * k[0, 4096 + 100]).sum(-1)
    assert (c_addr > 0.6).all() and (c_free.abs() < 0.4).all()   # noise norm 0.05*sqrt(128)


def test_decode_steps():
    w = inputs.WORKLOADS["decode"].with_(B=4, H=2)
    s = inputs.make_decode_steps(w, 3)
    assert s["q"].shape == (3, 4, 2, 128) and s["beta"].shape == (3, 4, 2)
    one = inputs.make_decode_step(w, 2, seqs=[1, 3])
    assert torch.equal(one["k"], s["k"][2, [1, 3]])
    S0 = inputs.decode_state(w)
    assert S0.shape == (4, 2, 128, 128)
