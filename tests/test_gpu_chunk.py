"""Chunked prefill (kda_chunk_fwd) on the GPU against the fp64 oracle."""
import time

import numpy as np
import pytest
import torch

import oracle
from linear_attention_sequence_chunk_amd import ChunkPlan, chunk_fwd, decode_step, inputs
from tests.parity import TOL, assert_close, cuda, max_err, to64

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)


def run_gpu(d, C, out_dtype=None):
    dg = cuda(d)
    o, S = chunk_fwd(dg["q"], dg["k"], dg["v"], dg["g"], dg["beta"], dg["S0"], chunk_size=C,
                     out_dtype=out_dtype)
    torch.cuda.synchronize()
    return o.cpu(), S.cpu()


def run_oracle(d, heads=None, cols=None):
    sel = lambda x: x if heads is None else x[:, :, heads]
    v = sel(d["v"])
    S0 = d["S0"]
    if heads is not None and S0 is not None:
        S0 = S0[:, heads]
    if cols is not None:
        v = v[..., cols]
        S0 = None if S0 is None else S0[..., cols]
    return oracle.recurrent(sel(d["q"]), sel(d["k"]), v, sel(d["g"]), sel(d["beta"]), S0)


def check(d, o, S, tol, heads=None, cols=None, tag=""):
    o_ref, S_ref = run_oracle(d, heads, cols)
    og = o if heads is None else o[:, :, heads]
    Sg = S if heads is None else S[:, heads]
    if cols is not None:
        og, Sg = og[..., cols], Sg[..., cols]
    eo = assert_close(f"{tag} o", og, o_ref, tol)
    es = assert_close(f"{tag} S", Sg, S_ref, tol)
    r_o, r_s = to64(o_ref), to64(S_ref)
    so = max(1.0, float(np.abs(r_o).max())) if r_o.size else 1.0
    ss = max(1.0, float(np.abs(r_s).max())) if r_s.size else 1.0
    _say(f"  {tag}: max err o {eo:.2e} (scale {so:.3g})  S {es:.2e} (scale {ss:.3g})")
    return eo, es


def test_tiny_fp32_workload():
    """B=1 H=2 T=256 d=64 C=64, fp32, 1e-4."""
    w = inputs.WORKLOADS["tiny"]
    _say("tiny fp32 workload")
    d = inputs.make_prefill(w)
    o, S = run_gpu(d, w.C)
    check(d, o, S, TOL[torch.float32], tag="tiny")


SHAPES = [(dk, dv) for dk in (64, 128) for dv in (64, 128)]


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
@pytest.mark.parametrize("C", [16, 32, 64, 128])
@pytest.mark.parametrize("dk,dv", SHAPES)
def test_shapes_ragged(dk, dv, C, dtype):
    """Several chunks plus a ragged tail, nonzero initial state, two batches
    (C = 128 runs as 64-token chunks for fp32 inputs and for dk = 128)."""
    _say(f"shape dk={dk} dv={dv} C={C} {dtype}")
    T = 3 * C + 11
    d = inputs.custom_prefill(C + dk + dv, 2, T, 3, dk, dv, dtype=dtype, s0_std=0.05)
    o, S = run_gpu(d, C)
    check(d, o, S, TOL[dtype], tag=f"dk{dk} dv{dv} C{C}")


@pytest.mark.parametrize("C", [16, 32, 64, 128])
def test_chunk_sizes_agree(C):
    """The chunk size is a performance knob: every C gives the oracle's result."""
    _say(f"chunk size agreement C={C}")
    d = inputs.custom_prefill(7, 1, 512, 2, 128, 128, dtype=torch.bfloat16, s0_std=0.01)
    o, S = run_gpu(d, C)
    check(d, o, S, TOL[torch.bfloat16], tag=f"C{C}")


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
def test_gate_edge_cases(dtype):
    """alpha = 0 on single channels, whole tokens and a whole chunk; alpha = 1
    runs; very fast gates (16-token sums far below -64, the term-by-term path);
    beta = 0 tokens."""
    _say(f"gate edge cases {dtype}")
    T, C = 320, 64
    d = inputs.custom_prefill(11, 1, T, 2, 64, 64, dtype=dtype, s0_std=0.1)
    g, beta = d["g"].clone(), d["beta"].clone()
    r = np.random.default_rng(3)
    idx = r.integers(0, T, 40)
    ch = r.integers(0, 64, 40)
    g[0, idx, 0, ch] = -float("inf")           # single (token, channel) clears
    g[0, 37, 1] = -float("inf")                 # a whole token
    g[0, 128:192, 0] = -float("inf")            # a whole chunk
    g[0, 200:230] = 0.0                         # alpha = 1 run
    g[0, 240:260, 1] = -9.0                     # fast gates: 16-token sum -144
    beta[0, 100:110] = 0.0
    d["g"], d["beta"] = g, beta
    o, S = run_gpu(d, C)
    # the kernel floors log-gates at -20: e^-20 ~ 2e-9 of the state leaks through
    check(d, o, S, TOL[dtype], tag="edges")


def test_empty_and_short_sequences():
    _say("T=0, T=1, T<C")
    for T in (0, 1, 5, 63):
        d = inputs.custom_prefill(13, 2, T, 2, 64, 64, dtype=torch.float32, s0_std=0.1) if T else None
        if T == 0:
            S0 = torch.randn(2, 2, 64, 64).cuda()
            z = torch.zeros(2, 0, 2, 64).cuda()
            o, S = chunk_fwd(z, z, z, z, torch.zeros(2, 0, 2).cuda(), S0, chunk_size=64)
            torch.cuda.synchronize()
            assert o.shape == (2, 0, 2, 64) and torch.equal(S, S0)
            o, S = chunk_fwd(z, z, z, z, torch.zeros(2, 0, 2).cuda(), None, chunk_size=64)
            torch.cuda.synchronize()
            assert torch.count_nonzero(S) == 0
            continue
        o, S = run_gpu(d, 64)
        check(d, o, S, 1e-4, tag=f"T{T}")


def test_out_dtype_fp32_and_in_place_state():
    _say("bf16 in / fp32 out, in-place state")
    d = inputs.custom_prefill(17, 1, 200, 2, 128, 128, dtype=torch.bfloat16, s0_std=0.05)
    dg = cuda(d)
    S_io = dg["S0"].clone()
    o, S = chunk_fwd(dg["q"], dg["k"], dg["v"], dg["g"], dg["beta"], S_io, chunk_size=64,
                     out_dtype=torch.float32, final_state=S_io)
    torch.cuda.synchronize()
    assert S.data_ptr() == S_io.data_ptr() and o.dtype == torch.float32
    check(d, o.cpu(), S.cpu(), TOL[torch.bfloat16], tag="inplace")


def test_deterministic_and_resumable():
    """Bitwise identical reruns; a split at a chunk boundary gives the same
    outputs and final state as one call (the state is the whole carried memory)."""
    _say("determinism and resume")
    d = inputs.custom_prefill(19, 2, 512, 2, 128, 128, dtype=torch.bfloat16, s0_std=0.02)
    o1, S1 = run_gpu(d, 64)
    o2, S2 = run_gpu(d, 64)
    assert torch.equal(o1, o2) and torch.equal(S1, S2)
    dg = cuda(d)
    cut = 192
    part = lambda x, a, b: x[:, a:b].contiguous()
    oa, Sa = chunk_fwd(*(part(dg[n], 0, cut) for n in ("q", "k", "v", "g", "beta")), dg["S0"], chunk_size=64)
    ob, Sb = chunk_fwd(*(part(dg[n], cut, 512) for n in ("q", "k", "v", "g", "beta")), Sa, chunk_size=64)
    torch.cuda.synchronize()
    assert torch.equal(torch.cat([oa, ob], 1).cpu(), o1) and torch.equal(Sb.cpu(), S1)


def test_value_column_permutation():
    """Value columns are independent: permuting v and S0 columns permutes o and
    S_T columns (bitwise, since every column is computed the same way)."""
    _say("value-column permutation")
    d = inputs.custom_prefill(23, 1, 256, 2, 128, 128, dtype=torch.float32, s0_std=0.05)
    o1, S1 = run_gpu(d, 64)
    perm = torch.randperm(128, generator=torch.Generator().manual_seed(0))
    d2 = dict(d); d2["v"] = d["v"][..., perm].contiguous(); d2["S0"] = d["S0"][..., perm].contiguous()
    o2, S2 = run_gpu(d2, 64)
    assert max_err(o2, o1[..., perm]) < 1e-6 and max_err(S2, S1[..., perm]) < 1e-6


def test_stages_match_fused_call():
    _say("intra + chain stages == kda_chunk_fwd")
    d = cuda(inputs.custom_prefill(29, 1, 300, 4, 128, 128, dtype=torch.bfloat16, s0_std=0.01))
    plan = ChunkPlan(d["q"], d["k"], d["v"], d["g"], d["beta"], d["S0"], chunk_size=64)
    o1, S1 = (x.clone() for x in plan.run())
    plan.o.zero_(); plan.final_state.zero_()
    plan.intra(); plan.chain()
    torch.cuda.synchronize()
    assert torch.equal(plan.o, o1) and torch.equal(plan.final_state, S1)


# ----------------------------------------------------------------- full-size workloads
@pytest.mark.parametrize("gates", ["tiny", "none", "scalar"], ids=["channel", "none", "scalar"])
def test_mid_workload(gates):
    """B=4 H=16 T=8192 d=128 C=64 bf16: the workload's own per-channel gates and
    the two gate sweeps (alpha = 1; one scalar gate per token and head) on the
    same q,k,v,beta.  The oracle checks every output and every final state: all
    64 (batch, head) sequences, all 128 value columns."""
    w = inputs.WORKLOADS["mid"]
    _say(f"mid workload gates={gates}: generating")
    d = inputs.make_prefill(w, gates=gates)
    _say(f"mid workload gates={gates}: GPU")
    o, S = run_gpu(d, w.C)
    _say(f"mid workload gates={gates}: oracle on all 64 sequences")
    t0 = time.perf_counter()
    check(d, o, S, TOL[torch.bfloat16], tag=f"mid/{gates}")
    _say(f"  oracle + comparison {time.perf_counter() - t0:.1f} s")


def test_mid_workload_bf16_log_gates():
    """The mid workload with every input in bf16, the log-gate too (the kernels
    widen it to fp32 on load): against the oracle on all 64 sequences (the oracle
    reads the stored bf16 gates exactly), and bitwise equal to the call with
    those same gate values handed over in fp32."""
    w = inputs.WORKLOADS["mid"]
    d = inputs.make_prefill(w)
    d["g"] = d["g"].to(torch.bfloat16)
    dg = cuda(d)
    o, S = chunk_fwd(dg["q"], dg["k"], dg["v"], dg["g"], dg["beta"], dg["S0"], chunk_size=w.C)
    o32, S32 = chunk_fwd(dg["q"], dg["k"], dg["v"], dg["g"].float(), dg["beta"], dg["S0"], chunk_size=w.C)
    torch.cuda.synchronize()
    assert torch.equal(o, o32) and torch.equal(S, S32), "bf16 gates differ from the same gates in fp32"
    check(d, o.cpu(), S.cpu(), TOL[torch.bfloat16], tag="mid/bf16 log-gates")


def test_long_workload():
    """B=1 H=32 T=65536 d=128 C=128 bf16, fast/slow channel gates, S0 ~ N(0,0.01);
    the oracle checks every output and final state of all 32 heads."""
    w = inputs.WORKLOADS["long"]
    _say("long workload: generating")
    d = inputs.make_prefill(w)
    _say("long workload: GPU")
    o, S = run_gpu(d, w.C)
    _say("long workload: oracle on all 32 heads")
    t0 = time.perf_counter()
    check(d, o, S, TOL[torch.bfloat16], tag="long")
    _say(f"  oracle + comparison {time.perf_counter() - t0:.1f} s")


def test_1m_token_workload():
    """B=1 H=16 T=1,048,576 d=128 C=64 bf16 (recurring address keys, fast/slow
    channel gates, S0 = 0).  With 16 heads the chain runs segment by segment
    (segment-affine form).
    (i) The final state and the outputs of the last 16,384 tokens: the oracle,
        on all 16 heads and all 128 value columns, runs from the GPU-produced
        state at T-16384 (the final state of a call over [0, T-16384)) and is
        compared with that split call's second part and with the single call.
    (ii) The single call equals the split call to the same bar (not bitwise:
        the two calls cut the sequence into different segments).
    (iii) The oracle follows 2 sampled heads over all 1,048,576 tokens on 4
        sampled value columns (columns of the recurrence are independent), from
        inputs regenerated on the host.
    (iv) The same call with the log-gates stored in bf16 (every input bf16):
        bitwise equal to the call with those gate values in fp32, and its final
        state and last 16,384 outputs against the oracle from the GPU state at
        T-16384 of the bf16-gate split call, as in (i)."""
    w = inputs.WORKLOADS["1m"]
    B, T, H, dk, dv = w.B, w.T, w.H, w.dk, w.dv
    dev = "cuda:0"
    heads, cols = [3, 12], [0, 37, 90, 127]
    tail = 16384
    T1 = T - tail
    q = torch.empty((B, T, H, dk), dtype=torch.bfloat16, device=dev)
    k = torch.empty_like(q)
    v = torch.empty((B, T, H, dv), dtype=torch.bfloat16, device=dev)
    g = torch.empty((B, T, H, dk), dtype=torch.float32, device=dev)
    beta = torch.empty((B, T, H), dtype=torch.float32, device=dev)
    host = {n: [] for n in ("q", "k", "v", "g", "beta")}
    piece = 1 << 16
    for t0 in range(0, T, piece):
        d = inputs.make_prefill(w, t0=t0, t1=t0 + piece)
        for n, dst in (("q", q), ("k", k), ("v", v), ("g", g), ("beta", beta)):
            dst[:, t0:t0 + piece].copy_(d[n])
            x = d[n][:, :, heads]
            host[n].append(x[..., cols] if n == "v" else x)
        if t0 % (1 << 18) == 0:
            _say(f"1m workload: inputs {t0 + piece}/{T}")
    host = {n: torch.cat(x, dim=1) for n, x in host.items()}
    tail_in = inputs.make_prefill(w, t0=T1, t1=T)         # all heads, the last 16,384 tokens

    _say("1m workload: single call")
    o, S = chunk_fwd(q, k, v, g, beta, None, chunk_size=w.C)
    _say("1m workload: split call")
    o1, S_mid = chunk_fwd(q[:, :T1], k[:, :T1], v[:, :T1], g[:, :T1], beta[:, :T1], None, chunk_size=w.C)
    o2, S2 = chunk_fwd(q[:, T1:], k[:, T1:], v[:, T1:], g[:, T1:], beta[:, T1:], S_mid, chunk_size=w.C)
    torch.cuda.synchronize()
    tol = TOL[torch.bfloat16]

    _say("1m workload: oracle on all 16 heads x 128 columns of the last 16,384 tokens from the GPU state")
    t0 = time.perf_counter()
    o_ref, S_ref = oracle.recurrent(tail_in["q"], tail_in["k"], tail_in["v"], tail_in["g"], tail_in["beta"],
                                    S_mid.cpu())
    _say(f"  oracle {time.perf_counter() - t0:.1f} s")
    e = [assert_close("1m tail o (split)", o2.cpu(), o_ref, tol), assert_close("1m S_T (split)", S2.cpu(), S_ref, tol),
         assert_close("1m tail o (single)", o[:, T1:].cpu(), o_ref, tol),
         assert_close("1m S_T (single)", S.cpu(), S_ref, tol)]
    _say("  1m tail: max err o {:.2e} S {:.2e} (split), o {:.2e} S {:.2e} (single)".format(*e))
    assert_close("1m single vs split o", o[:, :T1].cpu(), o1.cpu(), tol)

    _say("1m workload: oracle on 2 heads x 4 columns, all tokens")
    o_ref, S_ref = oracle.recurrent(host["q"], host["k"], host["v"], host["g"], host["beta"], None)
    og = o[:, :, heads][..., cols].cpu()
    Sg = S[:, heads][..., cols].cpu()
    eo = assert_close("1m o", og, o_ref, tol)
    es = assert_close("1m S", Sg, S_ref, tol)
    _say(f"  1m: max err o {eo:.2e}  S {es:.2e}")

    _say("1m workload: bf16 log-gates")
    del o, S, o1, o2, S2
    gb = g.to(torch.bfloat16)
    ob, Sb = chunk_fwd(q, k, v, gb, beta, None, chunk_size=w.C)
    ob32, Sb32 = chunk_fwd(q, k, v, gb.float(), beta, None, chunk_size=w.C)
    torch.cuda.synchronize()
    assert torch.equal(ob, ob32) and torch.equal(Sb, Sb32), "bf16 gates differ from the same gates in fp32"
    del ob32, Sb32
    _, Sb_mid = chunk_fwd(q[:, :T1], k[:, :T1], v[:, :T1], gb[:, :T1], beta[:, :T1], None, chunk_size=w.C)
    torch.cuda.synchronize()
    o_ref, S_ref = oracle.recurrent(tail_in["q"], tail_in["k"], tail_in["v"], tail_in["g"].to(torch.bfloat16),
                                    tail_in["beta"], Sb_mid.cpu())
    e = [assert_close("1m bf16-gate tail o", ob[:, T1:].cpu(), o_ref, tol),
         assert_close("1m bf16-gate S_T", Sb.cpu(), S_ref, tol)]
    _say("  1m bf16 log-gates, tail: max err o {:.2e} S {:.2e}".format(*e))


def test_decode_steps_match_prefill():
    """T consecutive kda_decode_step calls and one kda_chunk_fwd over the same
    sequence reach the same outputs and state (both are also checked against
    the oracle)."""
    d = inputs.custom_prefill(31, 2, 96, 3, 128, 128, dtype=torch.bfloat16, s0_std=0.05)
    dg = cuda(d)
    o_c, S_c = chunk_fwd(dg["q"], dg["k"], dg["v"], dg["g"], dg["beta"], dg["S0"], chunk_size=64)
    S = dg["S0"].clone()
    o_d = torch.empty_like(o_c)
    for t in range(d["q"].shape[1]):
        o_d[:, t] = decode_step(dg["q"][:, t].contiguous(), dg["k"][:, t].contiguous(),
                                dg["v"][:, t].contiguous(), dg["g"][:, t].contiguous(),
                                dg["beta"][:, t].contiguous(), S)
    torch.cuda.synchronize()
    check(d, o_d.cpu(), S.cpu(), TOL[torch.bfloat16], tag="decode x T")
    check(d, o_c.cpu(), S_c.cpu(), TOL[torch.bfloat16], tag="prefill")
    assert_close("decode vs prefill o", o_d.cpu(), o_c.cpu(), TOL[torch.bfloat16])
    assert_close("decode vs prefill S", S.cpu(), S_c.cpu(), TOL[torch.bfloat16])
