"""Backward pass through the fused pre-processing (kda_chunk_bwd_pre) on the GPU.

The gradients of the raw inputs (q and k rows before L2 normalisation, the gate
pre-activation a of the log-gate -softplus(a), fp32 or bf16 gate tensors) are
checked against the oracle: its fp64 adjoint of the pre-processed inputs,
followed by the vector-Jacobian products of the two steps
(oracle.l2_normalize_vjp, oracle.gate_softplus_vjp).  Raw rows with scales
0.05..20 and zero rows; both gate layouts; each flag alone and all together."""
import numpy as np
import pytest
import torch

import oracle
from linear_attention_sequence_chunk_amd import chunk_bwd
from tests.parity import assert_close
from tests.test_gpu_pre import _raw

pytestmark = pytest.mark.gpu

BWD_TOL = {torch.float32: 1e-4, torch.bfloat16: 2e-2}


def _say(m):
    print(m, flush=True)


def _case(dk, dv, C, dtype, layout, gdtype, qk, sp, seed, B=2, H=2, T=None):
    T = 2 * C + 9 if T is None else T
    d = _raw(seed, (B, T), H, dk, dv, dtype, gdtype, layout, zero_rows=True)
    # the tensors as the call takes them: raw where a flag applies, else pre-processed
    if qk:
        q_in, k_in = d["q"], d["k"]
    else:
        q_in = torch.tensor(oracle.l2_normalize(d["q"]), dtype=torch.float32).to(dtype)
        k_in = torch.tensor(oracle.l2_normalize(d["k"]), dtype=torch.float32).to(dtype)
    g_in = d["a"] if sp else torch.tensor(oracle.gate_softplus(d["a"]), dtype=torch.float32).to(gdtype)
    # the oracle's forward inputs
    qn = oracle.l2_normalize(q_in) if qk else oracle.to_f64(q_in)
    kn = oracle.l2_normalize(k_in) if qk else oracle.to_f64(k_in)
    g = oracle.gate_softplus(g_in) if sp else oracle.to_f64(g_in)
    if layout == "head":
        g = np.ascontiguousarray(np.broadcast_to(g[..., None], qn.shape))
    rs = np.random.default_rng(seed + 500)
    dO = torch.tensor(rs.standard_normal((B, T, H, dv)), dtype=torch.float32)
    dST = torch.tensor(rs.standard_normal((B, H, dk, dv)), dtype=torch.float32)

    dev = "cuda:0"
    got = chunk_bwd(q_in.to(dev), k_in.to(dev), d["v"].to(dev), g_in.to(dev), d["beta"].to(dev), dO.to(dev),
                    d["S0"].to(dev), dST.to(dev), chunk_size=C, gate_layout=layout, qk_l2norm=qk,
                    gate_act="softplus" if sp else None)
    torch.cuda.synchronize()
    got = {k: None if v is None else v.cpu() for k, v in got.items()}

    ref = oracle.backward(qn, kn, d["v"], g, d["beta"], d["S0"], dO, dST)
    want = dict(ref)
    if qk:
        want["dq"] = oracle.l2_normalize_vjp(q_in, ref["dq"])
        want["dk"] = oracle.l2_normalize_vjp(k_in, ref["dk"])
    dg = ref["dg"].sum(-1) if layout == "head" else ref["dg"]
    want["dg"] = oracle.gate_softplus_vjp(g_in, dg) if sp else dg
    tol = BWD_TOL[dtype]
    errs = {n: assert_close(f"{n}", got[n], want[n], tol) for n in ("dq", "dk", "dv", "dbeta", "dS0", "dg")}
    # rows that are zero before normalisation get no gradient
    if qk:
        zq = (q_in.float().reshape(-1, dk).abs().sum(-1) == 0)
        assert zq.any() and torch.all(got["dq"].reshape(-1, dk)[zq] == 0)
    _say(f"  dk={dk} dv={dv} C={C} {layout} qk={qk} softplus={sp} gate {gdtype}: "
         + "  ".join(f"{k} {v:.2e}" for k, v in errs.items()))


@pytest.mark.parametrize("dk,dv,C,dtype,layout,gdtype", [
    (128, 128, 64, torch.bfloat16, "channel", torch.bfloat16),
    (128, 128, 64, torch.bfloat16, "head", torch.float32),
    (64, 64, 32, torch.float32, "channel", torch.float32),
    (128, 64, 16, torch.float32, "channel", torch.bfloat16),
    (64, 128, 64, torch.float32, "head", torch.bfloat16)])
def test_backward_pre_all_flags(dk, dv, C, dtype, layout, gdtype):
    _say(f"backward pre dk={dk} dv={dv} C={C} {dtype} {layout} gate {gdtype}")
    _case(dk, dv, C, dtype, layout, gdtype, True, True, seed=dk + dv + C)


@pytest.mark.parametrize("qk,sp,gdtype", [(True, False, torch.float32), (False, True, torch.float32),
                                          (False, False, torch.bfloat16), (True, False, torch.bfloat16)])
def test_backward_pre_one_flag_at_a_time(qk, sp, gdtype):
    _say(f"backward pre qk={qk} softplus={sp} gate {gdtype}")
    _case(64, 64, 32, torch.float32, "channel", gdtype, qk, sp, seed=11)


def test_backward_pre_short_and_no_gate():
    """A single partial chunk; and no gates (the gate flags do nothing)."""
    _say("backward pre short / no gate")
    _case(128, 128, 64, torch.bfloat16, "channel", torch.bfloat16, True, True, seed=12, T=7)
    dev = "cuda:0"
    d = _raw(13, (1, 40), 2, 64, 64, torch.float32, torch.float32, "channel", zero_rows=False)
    dO = torch.randn((1, 40, 2, 64), generator=torch.Generator().manual_seed(3))
    got = chunk_bwd(d["q"].to(dev), d["k"].to(dev), d["v"].to(dev), None, d["beta"].to(dev), dO.to(dev),
                    chunk_size=32, gate_layout="none", qk_l2norm=True, gate_act="softplus")
    torch.cuda.synchronize()
    qn, kn = oracle.l2_normalize(d["q"]), oracle.l2_normalize(d["k"])
    ref = oracle.backward(qn, kn, d["v"], np.zeros_like(qn), d["beta"], None, dO, None)
    assert got["dg"] is None
    assert_close("no-gate dq", got["dq"].cpu(), oracle.l2_normalize_vjp(d["q"], ref["dq"]), 1e-4)
    assert_close("no-gate dk", got["dk"].cpu(), oracle.l2_normalize_vjp(d["k"], ref["dk"]), 1e-4)
    assert_close("no-gate dv", got["dv"].cpu(), ref["dv"], 1e-4)


def test_backward_pre_gate_alignment_and_odd_counts():
    """Per-head bf16 pre-activations given at element alignment only (a view two
    bytes into a buffer), and a count of gate values that is not a multiple of 8:
    the one-value-per-lane forms, which must agree bitwise with the eight-per-lane
    ones on the same values, and with the oracle."""
    _say("backward pre: gate alignment / odd counts")
    dev = "cuda:0"
    for T in (40, 37):                                    # 2*40*3 values: multiple of 8; 2*37*3: not
        d = _raw(70 + T, (2, T), 3, 64, 64, torch.float32, torch.bfloat16, "head", zero_rows=False)
        rs = np.random.default_rng(T)
        dO = torch.tensor(rs.standard_normal((2, T, 3, 64)), dtype=torch.float32)
        buf = torch.empty(d["a"].numel() + 1, dtype=torch.bfloat16)
        buf[1:] = d["a"].reshape(-1)
        a_mis = buf.to(dev)[1:].view(d["a"].shape)        # 2-byte aligned
        assert a_mis.data_ptr() % 16 != 0
        args = [d["q"].to(dev), d["k"].to(dev), d["v"].to(dev)]
        kw = dict(chunk_size=32, gate_layout="head", qk_l2norm=True, gate_act="softplus")
        got = chunk_bwd(*args, a_mis, d["beta"].to(dev), dO.to(dev), d["S0"].to(dev), **kw)
        ref = chunk_bwd(*args, d["a"].to(dev), d["beta"].to(dev), dO.to(dev), d["S0"].to(dev), **kw)
        torch.cuda.synchronize()
        for n in ("dq", "dk", "dv", "dbeta", "dS0", "dg"):
            assert torch.equal(got[n], ref[n]), n
        qn, kn = oracle.l2_normalize(d["q"]), oracle.l2_normalize(d["k"])
        g = oracle.gate_softplus(d["a"])
        g = np.ascontiguousarray(np.broadcast_to(g[..., None], qn.shape))
        o = oracle.backward(qn, kn, d["v"], g, d["beta"], d["S0"], dO, None)
        assert_close(f"T={T} dq", got["dq"].cpu(), oracle.l2_normalize_vjp(d["q"], o["dq"]), 1e-4)
        assert_close(f"T={T} dg", got["dg"].cpu(), oracle.gate_softplus_vjp(d["a"], o["dg"].sum(-1)), 1e-4)
