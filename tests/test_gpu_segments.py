"""The segment-affine chain on the GPU: long sequences with few (sequence, head)
pairs, where the sequential chain alone would occupy only a few CUs.

Each sequence is cut into segments whose affine maps S -> M S + E are composed
first; every segment then runs from its true start state.  That regroups the
chunk recurrence (chunk paragraph of the KimiK3 essay; sections 十五 and 十六 of
the explainer: the state after a chunk is an affine function of the state
before it), so the result is the oracle's up to rounding.  Checked here: every
output and final state against the fp64 oracle, a packed call on the same
tokens (packed batches run the plain sequential chain) at the same bar,
bitwise reruns and an in-place final state."""
import numpy as np
import pytest
import torch

import oracle
from linear_attention_sequence_chunk_amd import _lib, chunk_fwd, chunk_fwd_varlen, inputs
from tests.parity import TOL, assert_close, cuda

pytestmark = pytest.mark.gpu

# B, H, T, dv, out dtype, gates, S0 std
CASES = [
    (1, 2, 16384 + 37, 128, torch.bfloat16, "tiny", 0.05),
    (2, 1, 12288 + 64, 64, torch.bfloat16, "tiny", 0.0),
    (1, 3, 12000, 128, torch.float32, "none", 0.02),       # alpha = 1: M is not damped by decay
    (1, 1, 10240 + 5, 128, torch.bfloat16, "scalar", 0.05),  # 161 chunks: the fewest segments (5)
    (3, 2, 12000, 128, torch.bfloat16, "long", 0.01),
]


def _segments(B, T, H, dv):
    return _lib.lib().kda_chunk_fwd_segments(B, T, H, 128, dv, _lib.BF16, 64)


@pytest.mark.parametrize("B,H,T,dv,out_dtype,gates,s0", CASES)
def test_segmented_chain(B, H, T, dv, out_dtype, gates, s0):
    nseg = _segments(B, T, H, dv)
    assert nseg > 1, nseg
    print(f"segments B={B} H={H} T={T} dv={dv} {out_dtype} gates={gates}: {nseg} segments", flush=True)
    d = inputs.custom_prefill(61 + T, B, T, H, 128, dv, dtype=torch.bfloat16, gates=gates, s0_std=s0)
    dg = cuda(d)
    o, S = chunk_fwd(dg["q"], dg["k"], dg["v"], dg["g"], dg["beta"], dg["S0"], chunk_size=64, out_dtype=out_dtype)
    o2, S2 = chunk_fwd(dg["q"], dg["k"], dg["v"], dg["g"], dg["beta"], dg["S0"], chunk_size=64, out_dtype=out_dtype)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(S, S2), "reruns differ"

    # in place: the final state overwrites the initial state
    if dg["S0"] is not None:
        S_io = dg["S0"].clone()
        o3, S3 = chunk_fwd(dg["q"], dg["k"], dg["v"], dg["g"], dg["beta"], S_io, chunk_size=64,
                           out_dtype=out_dtype, final_state=S_io)
        torch.cuda.synchronize()
        assert torch.equal(o3, o) and torch.equal(S3, S), "in-place call differs"

    # the plain sequential chain on the same tokens: one packed batch of the B rows
    pk = lambda x: x.reshape((B * T,) + tuple(x.shape[2:])).contiguous()
    cu = torch.arange(0, B * T + 1, T, dtype=torch.int32, device="cuda:0")
    op, Sp = chunk_fwd_varlen(pk(dg["q"]), pk(dg["k"]), pk(dg["v"]), pk(dg["g"]), pk(dg["beta"]), cu,
                              dg["S0"], chunk_size=64, out_dtype=out_dtype)
    torch.cuda.synchronize()

    o_ref, S_ref = oracle.recurrent(d["q"], d["k"], d["v"], d["g"], d["beta"], d["S0"])
    tol = TOL[torch.bfloat16]
    eo = assert_close("o", o.cpu(), o_ref, tol)
    es = assert_close("S", S.cpu(), S_ref, tol)
    eop = assert_close("o (sequential chain)", op.cpu().reshape(o.shape), o_ref, tol)
    esp = assert_close("S (sequential chain)", Sp.cpu(), S_ref, tol)
    assert_close("o segmented vs sequential", o.cpu(), op.cpu().reshape(o.shape), tol)
    assert_close("S segmented vs sequential", S.cpu(), Sp.cpu(), tol)
    print(f"  segmented: o {eo:.2e} S {es:.2e};  sequential: o {eop:.2e} S {esp:.2e}", flush=True)


@pytest.mark.parametrize("seed", range(6))
def test_segmented_chain_random(seed):
    """Seeded random shapes that run in segments, with every gate layout and the
    fused pre-processing (raw q, k and a softplus pre-activation): outputs and
    final states against the oracle, on all heads and columns."""
    r = np.random.default_rng(400 + seed)
    B, H = int(r.integers(1, 3)), int(r.integers(1, 4))
    dv = int(r.choice([64, 128]))
    T = int(r.integers(64 * 160, 64 * 256)) + int(r.integers(0, 64))
    layout = ["channel", "head", "none"][seed % 3]
    pre = seed >= 3
    nseg = _segments(B, T, H, dv)
    assert nseg > 1
    print(f"random segments seed={seed}: B={B} H={H} T={T} dv={dv} gates={layout} pre={pre}: {nseg} segments",
          flush=True)
    d = inputs.custom_prefill(500 + seed, B, T, H, 128, dv, dtype=torch.bfloat16,
                              gates={"channel": "tiny", "head": "scalar", "none": "none"}[layout], s0_std=0.03)
    q, k, g = d["q"], d["k"], d["g"]
    if pre:
        # raw rows of varied scale, and the pre-activation whose -softplus is the gate
        sc = torch.tensor(r.uniform(0.2, 5.0, (B, T, H, 1)), dtype=torch.float32)
        q = (q.float() * sc).to(torch.bfloat16)
        k = (k.float() * sc.flip(1)).to(torch.bfloat16)
        a = torch.log(torch.expm1(-g.double())).float()
        g_in = a
    else:
        g_in = g
    if layout == "head":
        g_in = g_in[..., 0].contiguous()
    dg = cuda({"q": q, "k": k, "v": d["v"], "g": None if layout == "none" else g_in, "beta": d["beta"],
               "S0": d["S0"]})
    o, S = chunk_fwd(dg["q"], dg["k"], dg["v"], dg["g"], dg["beta"], dg["S0"], chunk_size=64, gate_layout=layout,
                     qk_l2norm=pre, gate_act="softplus" if pre else None)
    torch.cuda.synchronize()
    qn = oracle.l2_normalize(q) if pre else q
    kn = oracle.l2_normalize(k) if pre else k
    if layout == "none":
        g_ref = np.zeros(tuple(q.shape))
    else:
        g_ref = oracle.gate_softplus(g_in) if pre else oracle.to_f64(g_in)
        if layout == "head":
            g_ref = np.ascontiguousarray(np.broadcast_to(g_ref[..., None], tuple(q.shape)))
    o_ref, S_ref = oracle.recurrent(qn, kn, d["v"], g_ref, d["beta"], d["S0"])
    eo = assert_close("o", o.cpu(), o_ref, TOL[torch.bfloat16])
    es = assert_close("S", S.cpu(), S_ref, TOL[torch.bfloat16])
    print(f"  max err o {eo:.2e} S {es:.2e}", flush=True)
