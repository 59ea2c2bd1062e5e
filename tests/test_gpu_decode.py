"""Decode step (kda_decode_step) on the GPU against the fp64 oracle."""
import numpy as np
import pytest
import torch

import oracle
from linear_attention_sequence_chunk_amd import decode_step, inputs
from tests.parity import TOL, assert_close, cuda, to64

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)


def _oracle_steps(q, k, v, g, beta, S0):
    """Oracle over a sequence of decode steps: inputs [steps, N, H, d] ->
    recurrence with T = steps, B = N."""
    tr = lambda x: to64(x).swapaxes(0, 1)          # [N, steps, H, d]
    return oracle.recurrent(tr(q), tr(k), tr(v), tr(g), tr(beta), S0=to64(S0))


@pytest.mark.parametrize("dk,dv", [(64, 64), (64, 128), (128, 64), (128, 128)])
@pytest.mark.parametrize("dtype,out_dtype", [(torch.float32, torch.float32),
                                             (torch.bfloat16, torch.bfloat16),
                                             (torch.bfloat16, torch.float32)])
def test_decode_small(dk, dv, dtype, out_dtype):
    _say(f"decode small dk={dk} dv={dv} {dtype}->{out_dtype}")
    w = inputs.WORKLOADS["decode"].with_(B=5, H=3, dk=dk, dv=dv, dtype="f32" if dtype == torch.float32 else "bf16")
    steps = 7
    d = inputs.make_decode_steps(w, steps, threads=4)
    S0 = inputs.decode_state(w)
    S = S0.cuda()
    dg = cuda(d)
    outs = []
    for s in range(steps):
        outs.append(decode_step(dg["q"][s], dg["k"][s], dg["v"][s], dg["g"][s], dg["beta"][s], S,
                                out_dtype=out_dtype))
    torch.cuda.synchronize()
    o_ref, S_ref = _oracle_steps(d["q"], d["k"], d["v"], d["g"], d["beta"], S0)
    o_gpu = torch.stack(outs).cpu().transpose(0, 1)
    tol = 1e-4 if (dtype == torch.float32 and out_dtype == torch.float32) else TOL[torch.bfloat16]
    assert_close("o", o_gpu, o_ref, tol)
    assert_close("S", S, S_ref, 1e-4)       # fp32 state, exact inputs: fp32 rounding only


def test_decode_alpha_zero_and_beta_zero():
    _say("decode alpha=0 / beta=0 special cases")
    w = inputs.WORKLOADS["decode"].with_(B=2, H=2, dtype="f32")
    d = inputs.make_decode_step(w, 0)
    S0 = inputs.decode_state(w)
    g = d["g"].clone(); g[0, 0] = -float("inf")            # clears (n=0, h=0)
    beta = d["beta"].clone(); beta[1, 1] = 0.0              # no write on (1, 1)
    S = S0.cuda()
    o = decode_step(d["q"].cuda(), d["k"].cuda(), d["v"].cuda(), g.cuda(), beta.cuda(), S).cpu()
    Sc = S.cpu()
    k00, v00, b00 = d["k"][0, 0].double(), d["v"][0, 0].double(), beta[0, 0].double()
    np.testing.assert_allclose(to64(Sc[0, 0]), to64(torch.outer(k00, b00 * v00)), atol=1e-6)
    a11 = d["g"][1, 1].double().exp()
    np.testing.assert_allclose(to64(Sc[1, 1]), to64(a11[:, None] * S0[1, 1].double()), atol=1e-7)
    q00 = d["q"][0, 0].double()
    np.testing.assert_allclose(to64(o[0, 0]), to64((q00 @ k00) * b00 * v00), atol=1e-6)


def test_decode_full_size_1000_steps():
    """256 sequences x 32 heads x 128x128 states, 1000 consecutive steps.  The
    oracle checks every one of the 8192 states after steps 1 and 10 and every
    output of the first 10 steps, and follows 12 sampled (sequence, head)
    states through all 1000 steps."""
    w = inputs.WORKLOADS["decode"]
    steps = w.steps
    _say(f"decode full size: generating {steps} steps of inputs")
    d = inputs.make_decode_steps(w, steps)
    S0 = inputs.decode_state(w)
    rs = np.random.default_rng(5)
    seqs = rs.choice(w.B, 12, replace=False)
    heads = rs.integers(0, w.H, 12)
    S = S0.cuda()
    dg = cuda(d)
    sel = (torch.as_tensor(seqs).cuda(), torch.as_tensor(heads).cuda())
    o_hist = torch.empty((steps, 12, w.dv), dtype=torch.bfloat16, device="cuda")
    snaps, full, o_first = {}, {}, []
    _say("decode full size: running 1000 steps")
    for s in range(steps):
        o = decode_step(dg["q"][s], dg["k"][s], dg["v"][s], dg["g"][s], dg["beta"][s], S)
        o_hist[s] = o[sel]
        if s < 10:
            o_first.append(o.cpu())
        if s + 1 in (1, 10):
            full[s + 1] = S.cpu()
        if s + 1 in (1, 10, 100, 1000):
            snaps[s + 1] = S[sel].cpu()
    torch.cuda.synchronize()
    _say("decode full size: oracle on all 8192 states, steps 1 and 10")
    for upto in (1, 10):
        o_ref, S_ref = _oracle_steps(d["q"][:upto], d["k"][:upto], d["v"][:upto], d["g"][:upto],
                                     d["beta"][:upto], S0)
        es = assert_close(f"all S@{upto}", full[upto], S_ref, TOL[torch.bfloat16])
        eo = assert_close(f"all o, steps 1..{upto}", torch.stack(o_first[:upto]).transpose(0, 1), o_ref,
                          TOL[torch.bfloat16])
        assert_close(f"all S@{upto} (fp32 path)", full[upto], S_ref, 1e-4)
        _say(f"  step {upto}: max err S {es:.2e}, o {eo:.2e} over 8192 states")
        del o_ref, S_ref
    del full
    _say("decode full size: oracle on sampled states")
    pick = lambda x: x[:, seqs, heads][:, :, None]           # [steps, 12, 1, d]
    S0s = S0[seqs, heads][:, None]
    for upto in (1, 10, 100, 1000):
        o_ref, S_ref = _oracle_steps(pick(d["q"][:upto]), pick(d["k"][:upto]), pick(d["v"][:upto]),
                                     pick(d["g"][:upto]), pick(d["beta"][:upto]), S0s)
        assert_close(f"S@{upto}", snaps[upto], S_ref[:, 0], TOL[torch.bfloat16])
    assert_close("o", o_hist.cpu().transpose(0, 1), o_ref[:, :, 0], TOL[torch.bfloat16])
    # the state path itself is fp32 end to end: much tighter than the bf16 bar
    assert_close("S@1000 (fp32 path)", snaps[1000], S_ref[:, 0], 1e-4)


@pytest.mark.parametrize("T", [1, 2, 5, 8])
@pytest.mark.parametrize("layout", ["channel", "head", "none"])
def test_decode_tokens(T, layout):
    """T tokens per call (kda_decode_tokens) equal T single steps bitwise, and the
    oracle over the same T-token sequences."""
    _tokens_case(T, layout, 128, 128)


@pytest.mark.parametrize("T,dk,dv", [(2, 64, 64), (3, 64, 128), (2, 128, 64), (4, 64, 64)])
def test_decode_tokens_head_sizes(T, dk, dv):
    """The same for the other head sizes (each workgroup shape of the several-token
    kernel: 512 threads for two tokens, 256 from three on)."""
    _tokens_case(T, "channel", dk, dv)


def _tokens_case(T, layout, dk, dv):
    from linear_attention_sequence_chunk_amd import decode_tokens
    w = inputs.WORKLOADS["decode"].with_(B=6, H=3, dk=dk, dv=dv)
    d = inputs.make_decode_steps(w, T)                    # [T, N, H, ...]
    S0 = inputs.decode_state(w)
    seq = lambda x: x.transpose(0, 1).contiguous()        # -> [N, T, H, ...]
    if layout == "head":
        g_ch = d["g"][..., :1].expand_as(d["g"]).contiguous()
        g_in = seq(d["g"][..., 0])
    elif layout == "none":
        g_ch, g_in = torch.zeros_like(d["g"]), None
    else:
        g_ch = d["g"]
        g_in = seq(d["g"])
    q, k, v, beta = seq(d["q"]), seq(d["k"]), seq(d["v"]), seq(d["beta"])
    S = S0.cuda()
    o = decode_tokens(q.cuda(), k.cuda(), v.cuda(), None if g_in is None else g_in.cuda(), beta.cuda(), S,
                      gate_layout=layout)
    Ss = S0.cuda()
    steps = []
    for t in range(T):
        gl = None if g_in is None else g_in[:, t].contiguous().cuda()
        steps.append(decode_step(d["q"][t].cuda(), d["k"][t].cuda(), d["v"][t].cuda(), gl,
                                 d["beta"][t].cuda(), Ss, gate_layout=layout))
    torch.cuda.synchronize()
    assert torch.equal(o, torch.stack(steps, dim=1)) and torch.equal(S, Ss)
    o_ref, S_ref = oracle.recurrent(q, k, v, seq(g_ch), beta, S0)
    assert_close(f"tokens T={T} {layout} o", o.cpu(), o_ref, TOL[torch.bfloat16])
    assert_close(f"tokens T={T} {layout} S", S.cpu(), S_ref, TOL[torch.bfloat16])


def test_decode_tokens_full_size():
    """The four-token call bench.py times, at full size (256 sequences x 32 heads):
    bitwise equal to four single steps on every state and output, and the oracle
    on 8 sampled (sequence, head) pairs."""
    from linear_attention_sequence_chunk_amd import decode_tokens
    w = inputs.WORKLOADS["decode"]
    T = 4
    _say("decode tokens full size")
    d = inputs.make_decode_steps(w, T)                    # [T, N, H, ...]
    S0 = inputs.decode_state(w)
    seq = lambda x: x.transpose(0, 1).contiguous()        # -> [N, T, H, ...]
    dg = cuda(d)
    S = S0.cuda()
    o = decode_tokens(seq(dg["q"]), seq(dg["k"]), seq(dg["v"]), seq(dg["g"]), seq(dg["beta"]), S)
    Ss = S0.cuda()
    steps = [decode_step(dg["q"][t], dg["k"][t], dg["v"][t], dg["g"][t], dg["beta"][t], Ss) for t in range(T)]
    torch.cuda.synchronize()
    assert torch.equal(o, torch.stack(steps, dim=1)) and torch.equal(S, Ss)
    rs = np.random.default_rng(9)
    seqs, heads = rs.choice(w.B, 8, replace=False), rs.integers(0, w.H, 8)
    pick = lambda x: x[:, seqs, heads][:, :, None]        # [T, 8, 1, d]
    o_ref, S_ref = _oracle_steps(pick(d["q"]), pick(d["k"]), pick(d["v"]), pick(d["g"]), pick(d["beta"]),
                                 S0[seqs, heads][:, None])
    assert_close("S sampled", S[seqs, heads].cpu(), S_ref[:, 0], TOL[torch.bfloat16])
    assert_close("o sampled", o[seqs, :, heads].cpu(), o_ref[:, :, 0], TOL[torch.bfloat16])   # [8, T, dv]
