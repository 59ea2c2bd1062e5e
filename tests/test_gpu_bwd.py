"""Backward pass (kda_chunk_bwd) on the GPU against the oracle's fp64 adjoint.

Gradients of L = sum(dO * o) + sum(dST * S_T) for every input; ragged lengths
(partial last chunk), several chunks, every supported chunk size, both input
dtypes, all gate layouts."""
import numpy as np
import pytest
import torch

import oracle
from linear_attention_sequence_chunk_amd import chunk_bwd, inputs
from tests.parity import assert_close, cuda

pytestmark = pytest.mark.gpu

# fp32 inputs: the fp32-path bar of 1e-4 x scale; bf16 inputs: 2e-2 x scale.  Gradients
# accumulate in fp32; the products over the value channels (and, for bf16 inputs with
# C >= 32, the reverse chain) run on bf16 MFMA with their fp32 operands split into
# bf16 hi + lo parts (about 16 significant bits); with bf16 inputs the forward stages
# that are re-run for the backward use bf16 MFMA operands (as in the forward pass)
BWD_TOL = {torch.float32: 1e-4, torch.bfloat16: 2e-2}


def _say(m):
    print(m, flush=True)


def _run(d, C, layout, dtype, seed, tag):
    rs = np.random.default_rng(seed)
    B, T, H, dk = d["q"].shape
    dv = d["v"].shape[-1]
    dO = torch.tensor(rs.standard_normal((B, T, H, dv)), dtype=torch.float32)
    dST = torch.tensor(rs.standard_normal((B, H, dk, dv)), dtype=torch.float32)
    if layout == "head":
        g_in = d["g"][..., 0].contiguous()
        g_ref = g_in[..., None].expand_as(d["g"]).contiguous()
    elif layout == "none":
        g_in, g_ref = None, torch.zeros_like(d["g"])
    else:
        g_in = g_ref = d["g"]
    dg = cuda(d)
    got = chunk_bwd(dg["q"], dg["k"], dg["v"], None if g_in is None else g_in.cuda(), dg["beta"],
                    dO.cuda(), dg["S0"], dST.cuda(), chunk_size=C, gate_layout=layout)
    torch.cuda.synchronize()
    ref = oracle.backward(d["q"], d["k"], d["v"], g_ref, d["beta"], d["S0"], dO, dST)
    tol = BWD_TOL[dtype]
    errs = {}
    for name in ("dq", "dk", "dv", "dbeta", "dS0"):
        errs[name] = assert_close(f"{tag} {name}", got[name].cpu(), ref[name], tol)
    if layout == "channel":
        errs["dg"] = assert_close(f"{tag} dg", got["dg"].cpu(), ref["dg"], tol)
    elif layout == "head":
        errs["dg"] = assert_close(f"{tag} dg", got["dg"].cpu(), ref["dg"].sum(-1), tol)
    else:
        assert got["dg"] is None
    _say(f"  {tag}: " + "  ".join(f"{k} {v:.2e}" for k, v in errs.items()))


@pytest.mark.parametrize("dk,dv,C,dtype", [(64, 64, 64, torch.float32), (64, 128, 32, torch.float32),
                                           (128, 64, 16, torch.float32), (128, 128, 64, torch.bfloat16),
                                           (128, 128, 32, torch.bfloat16), (64, 64, 16, torch.bfloat16),
                                           (64, 128, 32, torch.bfloat16), (128, 64, 64, torch.bfloat16),
                                           (128, 128, 128, torch.bfloat16), (64, 64, 128, torch.float32),
                                           (64, 128, 128, torch.bfloat16)])
def test_backward_shapes(dk, dv, C, dtype):
    T = 3 * C + 11
    _say(f"backward dk={dk} dv={dv} C={C} {dtype} T={T}")
    d = inputs.custom_prefill(70 + C + dk + dv, 2, T, 2, dk, dv, dtype=dtype, s0_std=0.05)
    _run(d, C, "channel", dtype, 1, f"bwd dk{dk} dv{dv} C{C}")


@pytest.mark.parametrize("layout", ["head", "none"])
def test_backward_gate_layouts(layout):
    d = inputs.custom_prefill(81, 1, 150, 3, 128, 128, dtype=torch.bfloat16,
                              gates="scalar" if layout == "head" else "none", s0_std=0.05)
    _run(d, 64, layout, torch.bfloat16, 2, f"bwd {layout}")


def test_backward_longer_sequence():
    """1024 tokens, 16 chunks of 64: the reverse chain over many chunks."""
    d = inputs.custom_prefill(83, 1, 1024, 4, 128, 128, dtype=torch.bfloat16, s0_std=0.02)
    _run(d, 64, "channel", torch.bfloat16, 3, "bwd T1024")


def test_backward_is_deterministic():
    d = cuda(inputs.custom_prefill(85, 1, 200, 2, 64, 64, dtype=torch.float32, s0_std=0.05))
    dO = torch.randn((1, 200, 2, 64), generator=torch.Generator().manual_seed(0)).cuda()
    a = chunk_bwd(d["q"], d["k"], d["v"], d["g"], d["beta"], dO, d["S0"], chunk_size=32)
    b = chunk_bwd(d["q"], d["k"], d["v"], d["g"], d["beta"], dO, d["S0"], chunk_size=32)
    torch.cuda.synchronize()
    for name in a:
        assert torch.equal(a[name], b[name]), name


@pytest.mark.parametrize("T,dk,dv,C,dtype", [(1, 128, 128, 64, torch.bfloat16), (5, 128, 128, 64, torch.bfloat16),
                                             (31, 64, 64, 32, torch.float32), (17, 64, 128, 16, torch.float32)])
def test_backward_short_sequences(T, dk, dv, C, dtype):
    """A single partial chunk (T < C), or a full one and a partial one."""
    d = inputs.custom_prefill(90 + T, 2, T, 3, dk, dv, dtype=dtype, s0_std=0.05)
    _run(d, C, "channel", dtype, 5, f"bwd T{T} C{C}")


def test_backward_empty_sequence():
    """T = 0: dS0 is dS_T, nothing else is written."""
    dk = dv = 64
    q = torch.zeros((2, 0, 3, dk), device="cuda")
    beta = torch.zeros((2, 0, 3), device="cuda")
    dO = torch.zeros((2, 0, 3, dv), device="cuda")
    dST = torch.randn((2, 3, dk, dv), generator=torch.Generator().manual_seed(1)).cuda()
    out = chunk_bwd(q, q, dO.clone(), q, beta, dO, None, dST, chunk_size=64)
    torch.cuda.synchronize()
    assert torch.equal(out["dS0"], dST)
    assert out["dq"].numel() == 0 and out["dg"].numel() == 0


def test_backward_strong_gates():
    """Log-gates ~ -U(0, 8): many 16-token blocks sum below -SAFE_SPAN (the
    term-by-term diagonal paths of the forward and the backward), and a few gates
    below the -20 floor (gradient 0 there; the oracle's exact value is ~e^g)."""
    import numpy as np
    B, T, H, dk, dv = 1, 200, 2, 128, 128
    d = inputs.custom_prefill(97, B, T, H, dk, dv, dtype=torch.float32, s0_std=0.05)
    g = -np.random.default_rng(6).uniform(0.0, 8.0, (B, T, H, dk))
    g[0, 40:42, 0, :5] = -30.0
    d["g"] = torch.tensor(g, dtype=torch.float32)
    _run(d, 64, "channel", torch.float32, 6, "bwd strong gates")


def test_backward_mid_workload_full():
    """The backward pass at the size bench.py times it (B=4, H=16, T=8192, d=128,
    C=64, bf16 q/k/v, per-channel gates): every gradient of every (batch, head)
    sequence against the oracle's fp64 adjoint, with a final-state cotangent as
    well, so that dS0 is checked too."""
    import time
    w = inputs.WORKLOADS["mid"]
    _say("backward mid workload: generating")
    d = inputs.make_prefill(w)
    rs = np.random.default_rng(8)
    dO = torch.tensor(rs.standard_normal((w.B, w.T, w.H, w.dv)), dtype=torch.float32)
    dST = torch.tensor(rs.standard_normal((w.B, w.H, w.dk, w.dv)), dtype=torch.float32)
    _say("backward mid workload: GPU")
    dg = cuda(d)
    got = chunk_bwd(dg["q"], dg["k"], dg["v"], dg["g"], dg["beta"], dO.cuda(), dg["S0"], dST.cuda(),
                    chunk_size=w.C)
    torch.cuda.synchronize()
    got = {k: (None if v is None else v.cpu()) for k, v in got.items()}
    del dg
    _say("backward mid workload: oracle on all 64 sequences")
    t0 = time.perf_counter()
    ref = oracle.backward(d["q"], d["k"], d["v"], d["g"], d["beta"], d["S0"], dO, dST)
    t1 = time.perf_counter()
    tol = BWD_TOL[torch.bfloat16]
    errs = {name: assert_close(f"bwd mid {name}", got[name], ref[name], tol)
            for name in ("dq", "dk", "dv", "dg", "dbeta", "dS0")}
    scales = {name: max(1.0, float(np.abs(ref[name]).max())) for name in errs}
    _say(f"  oracle {t1 - t0:.1f} s;  max abs err / scale: " +
         "  ".join(f"{k} {v:.2e}/{scales[k]:.3g}" for k, v in errs.items()))
