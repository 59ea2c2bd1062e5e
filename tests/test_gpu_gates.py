"""Gate layouts (kda_gate_layout_t) on the GPU: one gate per head (Gated
DeltaNet) and no gate (DeltaNet), for prefill and decode.  Each is checked
against the fp64 oracle (which takes the per-channel gate: the per-head gate
broadcast over channels, or zeros) and bitwise against the per-channel call fed
that same broadcast gate."""
import pytest
import torch

from linear_attention_sequence_chunk_amd import chunk_fwd, decode_step, inputs
from tests.parity import TOL, assert_close, cuda
from tests.test_gpu_chunk import check

pytestmark = pytest.mark.gpu

# (dk, dv, C, dtype): the hot configuration and generic ones
CONFIGS = [(128, 128, 64, torch.bfloat16), (128, 64, 64, torch.bfloat16), (64, 64, 32, torch.float32),
           (128, 128, 128, torch.bfloat16), (64, 128, 16, torch.float32)]


def _layout_inputs(d, layout):
    """(g for the layout under test, the equivalent per-channel g)."""
    if layout == "head":
        gh = d["g"][..., 0].contiguous()                  # scalar recipe: equal over channels
        assert torch.equal(d["g"], gh[..., None].expand_as(d["g"]))
        return gh, d["g"]
    return None, torch.zeros_like(d["g"])


@pytest.mark.parametrize("layout", ["head", "none"])
@pytest.mark.parametrize("dk,dv,C,dtype", CONFIGS)
def test_prefill_gate_layouts(layout, dk, dv, C, dtype):
    T = 3 * C + 17
    d = inputs.custom_prefill(40 + dk + dv + C, 2, T, 3, dk, dv, dtype=dtype,
                              gates="scalar" if layout == "head" else "none", s0_std=0.05)
    g_layout, g_channel = _layout_inputs(d, layout)
    dg = cuda(d)
    gl = None if g_layout is None else g_layout.cuda()
    o, S = chunk_fwd(dg["q"], dg["k"], dg["v"], gl, dg["beta"], dg["S0"], chunk_size=C, gate_layout=layout)
    o_c, S_c = chunk_fwd(dg["q"], dg["k"], dg["v"], g_channel.cuda(), dg["beta"], dg["S0"], chunk_size=C)
    torch.cuda.synchronize()
    assert torch.equal(o, o_c) and torch.equal(S, S_c), "layout differs from the per-channel call"
    ref = dict(d); ref["g"] = g_channel
    check(ref, o.cpu(), S.cpu(), TOL[dtype], tag=f"{layout} dk{dk} dv{dv} C{C}")


@pytest.mark.parametrize("layout", ["head", "none"])
def test_decode_gate_layouts(layout):
    w = inputs.WORKLOADS["decode"].with_(B=8, H=4)
    steps = 6
    d = inputs.make_decode_steps(w, steps)
    S0 = inputs.decode_state(w)
    if layout == "head":
        g_layout = d["g"][..., 0].contiguous()             # [steps, N, H]
        g_channel = g_layout[..., None].expand_as(d["g"]).contiguous()
    else:
        g_layout, g_channel = None, torch.zeros_like(d["g"])
    dg = cuda(d)
    S, Sc = S0.cuda(), S0.cuda()
    outs, outs_c = [], []
    for s in range(steps):
        gl = None if g_layout is None else g_layout[s].cuda()
        outs.append(decode_step(dg["q"][s], dg["k"][s], dg["v"][s], gl, dg["beta"][s], S, gate_layout=layout))
        outs_c.append(decode_step(dg["q"][s], dg["k"][s], dg["v"][s], g_channel[s].cuda(), dg["beta"][s], Sc))
    torch.cuda.synchronize()
    o, o_c = torch.stack(outs), torch.stack(outs_c)
    assert torch.equal(o, o_c) and torch.equal(S, Sc)
    # oracle: the steps as a sequence of length `steps` per (n, h)
    seq = lambda x: x.transpose(0, 1).contiguous()         # [N, steps, H, ...]
    ref = {"q": seq(d["q"]), "k": seq(d["k"]), "v": seq(d["v"]), "g": seq(g_channel),
           "beta": seq(d["beta"]), "S0": S0}
    check(ref, seq(o.cpu()), S.cpu(), TOL[torch.bfloat16], tag=f"decode {layout}")


@pytest.mark.parametrize("dk,dv,C,dtype", [(128, 128, 64, torch.bfloat16), (64, 64, 32, torch.float32),
                                           (128, 64, 16, torch.float32)])
def test_prefill_without_decay_every_chunk_count(dk, dv, C, dtype):
    """alpha = 1 (no gate): nothing decays, so an error anywhere in the chain of
    states stays visible to the end; every chunk count 1..11 (all positions of the
    last chunk within the chain kernels' prefetch rounds), full and partial."""
    for nc in range(1, 12):
        for T in (nc * C, nc * C - 5):
            d = inputs.custom_prefill(200 + nc, 1, T, 2, dk, dv, dtype=dtype, gates="none", s0_std=0.05)
            dg = cuda(d)
            o, S = chunk_fwd(dg["q"], dg["k"], dg["v"], None, dg["beta"], dg["S0"], chunk_size=C, gate_layout="none")
            torch.cuda.synchronize()
            ref = dict(d)
            ref["g"] = torch.zeros_like(d["g"])
            check(ref, o.cpu(), S.cpu(), TOL[dtype], tag=f"no decay dk{dk} dv{dv} C{C} T{T}")


@pytest.mark.parametrize("layout", ["head", "none"])
def test_prefill_gate_layouts_mid_workload_full(layout):
    """The gate layouts at the size bench.py times them (B=4, H=16, T=8192,
    d=128, C=64, bf16): one gate per (token, head) given as [B,T,H], and no gate;
    every output and final state of all 64 sequences against the oracle, and
    bitwise against the per-channel call fed the broadcast gate."""
    w = inputs.WORKLOADS["mid"]
    d = inputs.make_prefill(w, gates="scalar" if layout == "head" else "none")
    g_layout, g_channel = _layout_inputs(d, layout)
    dg = cuda(d)
    gl = None if g_layout is None else g_layout.cuda()
    o, S = chunk_fwd(dg["q"], dg["k"], dg["v"], gl, dg["beta"], dg["S0"], chunk_size=w.C, gate_layout=layout)
    o_c, S_c = chunk_fwd(dg["q"], dg["k"], dg["v"], g_channel.cuda(), dg["beta"], dg["S0"], chunk_size=w.C)
    torch.cuda.synchronize()
    assert torch.equal(o, o_c) and torch.equal(S, S_c), "layout differs from the per-channel call"
    ref = dict(d); ref["g"] = g_channel
    check(ref, o.cpu(), S.cpu(), TOL[torch.bfloat16], tag=f"mid {layout}")
