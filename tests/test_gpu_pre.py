"""Fused pre-processing on the GPU (kda_chunk_fwd_pre, kda_chunk_intra_pre,
kda_decode_tokens_pre): raw q and k normalised inside the kernels, the log-gate
given as a pre-activation a (log-gate -softplus(a)), fp32 or bf16 gates.  Each is
checked against the fp64 oracle fed the pre-processed inputs
(oracle.l2_normalize, oracle.gate_softplus): ragged lengths, several chunks, the
hot and generic kernels, both gate layouts, zero rows."""
import numpy as np
import pytest
import torch

import oracle
from linear_attention_sequence_chunk_amd import ChunkPlan, chunk_fwd, decode_tokens
from tests.parity import TOL, assert_close

pytestmark = pytest.mark.gpu


def _say(m):
    print(m, flush=True)


def _raw(seed, lead, H, dk, dv, dtype, gdtype, layout, zero_rows=False):
    """Unnormalised q, k (row scales 0.05..20), gate pre-activations a ~ N(0,1) + 2,
    v ~ N(0,1), beta in (0, 1), S0 ~ N(0, 0.05) (one state per leading index 0)."""
    rs = np.random.default_rng(seed)
    shp = tuple(lead) + (H,)
    q = rs.standard_normal(shp + (dk,)) * rs.uniform(0.05, 20.0, shp + (1,))
    k = rs.standard_normal(shp + (dk,)) * rs.uniform(0.05, 20.0, shp + (1,))
    if zero_rows:
        k.reshape(-1, dk)[::7] = 0.0
        q.reshape(-1, dk)[::11] = 0.0
    v = rs.standard_normal(shp + (dv,))
    a = rs.standard_normal(shp + ((dk,) if layout == "channel" else ())) + 2.0
    beta = rs.uniform(0.05, 0.95, shp)
    S0 = rs.standard_normal((lead[0], H, dk, dv)) * 0.05
    t = lambda x, dt: torch.tensor(x, dtype=torch.float32).to(dt)
    return dict(q=t(q, dtype), k=t(k, dtype), v=t(v, dtype), a=t(a, gdtype), beta=t(beta, torch.float32),
                S0=t(S0, torch.float32))


def _oracle_inputs(d, layout):
    q, k = oracle.l2_normalize(d["q"]), oracle.l2_normalize(d["k"])
    g = oracle.gate_softplus(d["a"])
    if layout == "head":
        g = np.ascontiguousarray(np.broadcast_to(g[..., None], q.shape))
    return q, k, g


CONFIGS = [(128, 128, 64, torch.bfloat16, "channel", torch.bfloat16),   # hot kernel, bf16 gate
           (128, 128, 64, torch.bfloat16, "channel", torch.float32),
           (128, 128, 64, torch.bfloat16, "head", torch.bfloat16),
           (128, 64, 32, torch.bfloat16, "channel", torch.bfloat16),     # generic kernels
           (64, 64, 64, torch.float32, "channel", torch.float32),
           (64, 128, 16, torch.float32, "channel", torch.bfloat16),
           (128, 128, 128, torch.bfloat16, "head", torch.float32)]


@pytest.mark.parametrize("dk,dv,C,dtype,layout,gdtype", CONFIGS)
def test_prefill_pre(dk, dv, C, dtype, layout, gdtype):
    B, H, T = 2, 3, 3 * C + 13
    d = _raw(dk + dv + C, (B, T), H, dk, dv, dtype, gdtype, layout, zero_rows=True)
    dg = {key: x.cuda() for key, x in d.items()}
    o, S = chunk_fwd(dg["q"], dg["k"], dg["v"], dg["a"], dg["beta"], dg["S0"], chunk_size=C,
                     gate_layout=layout, qk_l2norm=True, gate_act="softplus")
    plan = ChunkPlan(dg["q"], dg["k"], dg["v"], dg["a"], dg["beta"], dg["S0"], chunk_size=C,
                     gate_layout=layout, qk_l2norm=True, gate_act="softplus")
    plan.intra()
    plan.chain()
    torch.cuda.synchronize()
    assert torch.equal(plan.o, o) and torch.equal(plan.final_state, S), "intra/chain split differs"
    q, k, g = _oracle_inputs(d, layout)
    o_ref, S_ref = oracle.recurrent(q, k, d["v"], g, d["beta"], d["S0"])
    tag = f"pre dk{dk} dv{dv} C{C} {layout} g:{str(gdtype)[6:]}"
    eo = assert_close(f"{tag} o", o.cpu(), o_ref, TOL[dtype])
    es = assert_close(f"{tag} S", S.cpu(), S_ref, TOL[dtype])
    _say(f"  {tag}: max err o {eo:.2e}  S {es:.2e}")


def test_prefill_pre_flags_one_at_a_time():
    """Each flag alone: normalisation only (log-gate given), activation only
    (q, k already unit)."""
    dk = dv = 128
    C, B, H, T = 64, 1, 2, 200
    d = _raw(7, (B, T), H, dk, dv, torch.bfloat16, torch.float32, "channel")
    dg = {key: x.cuda() for key, x in d.items()}
    q, k, g = _oracle_inputs(d, "channel")
    g_t = torch.tensor(g, dtype=torch.float32).cuda()
    o, S = chunk_fwd(dg["q"], dg["k"], dg["v"], g_t, dg["beta"], dg["S0"], chunk_size=C, qk_l2norm=True)
    o_ref, S_ref = oracle.recurrent(q, k, d["v"], g, d["beta"], d["S0"])
    assert_close("norm only o", o.cpu(), o_ref, 2e-2)
    assert_close("norm only S", S.cpu(), S_ref, 2e-2)
    qb = torch.tensor(q).to(torch.bfloat16).cuda()
    kb = torch.tensor(k).to(torch.bfloat16).cuda()
    o2, S2 = chunk_fwd(qb, kb, dg["v"], dg["a"], dg["beta"], dg["S0"], chunk_size=C, gate_act="softplus")
    o2_ref, S2_ref = oracle.recurrent(qb.cpu(), kb.cpu(), d["v"], g, d["beta"], d["S0"])
    assert_close("softplus only o", o2.cpu(), o2_ref, 2e-2)
    assert_close("softplus only S", S2.cpu(), S2_ref, 2e-2)


@pytest.mark.parametrize("T,dtype,layout,gdtype", [(1, torch.bfloat16, "channel", torch.bfloat16),
                                                   (3, torch.bfloat16, "head", torch.bfloat16),
                                                   (4, torch.float32, "channel", torch.float32)])
def test_decode_pre(T, dtype, layout, gdtype):
    N, H, dk, dv = 6, 4, 128, 128
    d = _raw(30 + T, (N, T), H, dk, dv, dtype, gdtype, layout, zero_rows=True)
    dg = {key: x.cuda() for key, x in d.items()}
    S = dg["S0"].clone()
    o = decode_tokens(dg["q"], dg["k"], dg["v"], dg["a"], dg["beta"], S, gate_layout=layout,
                      qk_l2norm=True, gate_act="softplus")
    torch.cuda.synchronize()
    q, k, g = _oracle_inputs(d, layout)
    o_ref, S_ref = oracle.recurrent(q, k, d["v"], g, d["beta"], d["S0"])   # [N,T,...] as [B,T,...]
    tag = f"decode pre T{T} {layout}"
    eo = assert_close(f"{tag} o", o.cpu(), o_ref, TOL[dtype])
    es = assert_close(f"{tag} S", S.cpu(), S_ref, TOL[dtype])
    _say(f"  {tag}: max err o {eo:.2e}  S {es:.2e}")


@pytest.mark.parametrize("T,dk,dv,layout,gdtype,sp,qk", [(2, 128, 128, "channel", torch.bfloat16, False, False),
                                                         (2, 64, 128, "head", torch.bfloat16, False, True),
                                                         (5, 64, 64, "channel", torch.bfloat16, True, False),
                                                         (1, 128, 64, "head", torch.float32, True, True),
                                                         (3, 128, 64, "channel", torch.bfloat16, False, True)])
def test_decode_gate_forms(T, dk, dv, layout, gdtype, sp, qk):
    """Decode over each gate storage the kernels read (fp32 or bf16, per channel or
    per head, log-gate or pre-activation), head sizes 64 and 128, one or several
    tokens per call; the flags one at a time."""
    N, H = 5, 3
    d = _raw(60 + T + dk, (N, T), H, dk, dv, torch.bfloat16, gdtype, layout, zero_rows=False)
    if not sp:                                            # a log-gate in (-3, 0), stored as given
        d["a"] = (-torch.nn.functional.softplus(d["a"].float())).to(gdtype)
    dg = {key: x.cuda() for key, x in d.items()}
    S = dg["S0"].clone()
    o = decode_tokens(dg["q"], dg["k"], dg["v"], dg["a"], dg["beta"], S, gate_layout=layout,
                      qk_l2norm=qk, gate_act="softplus" if sp else None)
    torch.cuda.synchronize()
    q = oracle.l2_normalize(d["q"]) if qk else oracle.to_f64(d["q"])
    k = oracle.l2_normalize(d["k"]) if qk else oracle.to_f64(d["k"])
    g = oracle.gate_softplus(d["a"]) if sp else oracle.to_f64(d["a"])
    if layout == "head":
        g = np.ascontiguousarray(np.broadcast_to(g[..., None], q.shape))
    o_ref, S_ref = oracle.recurrent(q, k, d["v"], g, d["beta"], d["S0"])
    tag = f"decode T{T} dk{dk} dv{dv} {layout} {gdtype} softplus={sp} norm={qk}"
    eo = assert_close(f"{tag} o", o.cpu(), o_ref, TOL[torch.bfloat16])
    es = assert_close(f"{tag} S", S.cpu(), S_ref, TOL[torch.bfloat16])
    _say(f"  {tag}: max err o {eo:.2e}  S {es:.2e}")


def test_prefill_pre_mid_workload_full():
    """The fused pre-processing at the size bench.py times it (B=4, H=16, T=8192,
    d=128, C=64): raw bf16 q and k (the workload's rows scaled by 0.2..5) and a
    bf16 gate pre-activation whose -softplus is the workload's log-gate; every
    output and final state of all 64 sequences against the oracle fed the
    pre-processed inputs."""
    from linear_attention_sequence_chunk_amd import inputs
    w = inputs.WORKLOADS["mid"]
    _say("pre mid workload: generating")
    d = inputs.make_prefill(w)
    rs = np.random.default_rng(12)
    sc = lambda: torch.tensor(rs.uniform(0.2, 5.0, (w.B, w.T, w.H, 1)), dtype=torch.float32)
    q = (d["q"].float() * sc()).to(torch.bfloat16)
    k = (d["k"].float() * sc()).to(torch.bfloat16)
    a = torch.log(torch.expm1(-d["g"].double())).to(torch.bfloat16)
    _say("pre mid workload: GPU")
    o, S = chunk_fwd(q.cuda(), k.cuda(), d["v"].cuda(), a.cuda(), d["beta"].cuda(),
                     None if d["S0"] is None else d["S0"].cuda(), chunk_size=w.C, qk_l2norm=True,
                     gate_act="softplus")
    torch.cuda.synchronize()
    _say("pre mid workload: oracle on all 64 sequences")
    o_ref, S_ref = oracle.recurrent(oracle.l2_normalize(q), oracle.l2_normalize(k), d["v"],
                                    oracle.gate_softplus(a), d["beta"], d["S0"])
    eo = assert_close("pre mid o", o.cpu(), o_ref, TOL[torch.bfloat16])
    es = assert_close("pre mid S", S.cpu(), S_ref, TOL[torch.bfloat16])
    _say(f"  pre mid: max err o {eo:.2e}  S {es:.2e}")
