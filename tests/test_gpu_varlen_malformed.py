"""Packed batches whose offsets break the rules (decreasing, overlapping, outside
[0, T]) on the GPU, forward and backward.

The library promises only that every access stays in bounds; on the device each
offset becomes the running maximum of the offsets so far, clamped to [0, T].
So the result is defined: sequence s covers tokens [m_s, m_{s+1}) with
m = min(T, running max(max(0, cu_seqlens))).  Each such sequence must equal a
fixed-length call on its tokens alone, bitwise, forward and backward."""
import numpy as np
import pytest
import torch

from linear_attention_sequence_chunk_amd import chunk_bwd, chunk_bwd_varlen, chunk_fwd, chunk_fwd_varlen, inputs

pytestmark = pytest.mark.gpu

CASES = [
    ("restart at zero", [0, 700, 0, 700]),
    ("decreasing and overlapping", [0, 300, 100, 500, 50, 700, 800]),
    ("outside [0, T]", [-40, 130, 2000, -5, 700]),
]


def _effective(cu, T):
    return np.minimum(T, np.maximum.accumulate(np.maximum(0, np.asarray(cu))))


@pytest.mark.parametrize("name,cu", CASES, ids=[c[0] for c in CASES])
@pytest.mark.parametrize("C", [64, 32])
def test_malformed_offsets_forward_and_backward(name, cu, C):
    T, H, dk, dv = 700, 2, 128, 128
    dtype = torch.bfloat16 if C == 64 else torch.float32
    print(f"malformed offsets '{name}' {cu} C={C}", flush=True)
    d = inputs.custom_prefill(41, 1, T, H, dk, dv, dtype=dtype, s0_std=0.05)
    dev = "cuda:0"
    N = len(cu) - 1
    S0 = torch.randn((N, H, dk, dv), generator=torch.Generator().manual_seed(3)) * 0.05
    p = {k: d[k][0].to(dev).contiguous() for k in ("q", "k", "v", "g", "beta")}
    cu_d = torch.tensor(cu, dtype=torch.int32, device=dev)
    o, S = chunk_fwd_varlen(p["q"], p["k"], p["v"], p["g"], p["beta"], cu_d, S0.to(dev), chunk_size=C)
    rs = np.random.default_rng(5)
    dO = torch.tensor(rs.standard_normal((T, H, dv)), dtype=torch.float32, device=dev)
    dST = torch.tensor(rs.standard_normal((N, H, dk, dv)), dtype=torch.float32, device=dev)
    grads = chunk_bwd_varlen(p["q"], p["k"], p["v"], p["g"], p["beta"], dO, cu_d, S0.to(dev), dST, chunk_size=C)
    torch.cuda.synchronize()

    m = _effective(cu, T)
    for s in range(N):
        a, b = int(m[s]), int(m[s + 1])
        s0 = S0[s:s + 1].to(dev)
        if b == a:
            assert torch.equal(S[s].cpu(), S0[s]), f"empty sequence {s}: final state is not its initial state"
            assert torch.equal(grads["dS0"][s], dST[s]), f"empty sequence {s}: dS0 is not dST"
            continue
        sl = {k: v[a:b][None].contiguous() for k, v in p.items()}
        oi, Si = chunk_fwd(sl["q"], sl["k"], sl["v"], sl["g"], sl["beta"], s0, chunk_size=C)
        own = chunk_bwd(sl["q"], sl["k"], sl["v"], sl["g"], sl["beta"], dO[a:b][None].contiguous(), s0,
                        dST[s:s + 1].contiguous(), chunk_size=C)
        torch.cuda.synchronize()
        assert torch.equal(o[a:b], oi[0]), f"sequence {s} [{a},{b}): o differs from its own call"
        assert torch.equal(S[s], Si[0]), f"sequence {s}: final state differs from its own call"
        for gname in ("dq", "dk", "dv", "dg", "dbeta"):
            assert torch.equal(grads[gname][a:b], own[gname][0]), f"sequence {s}: {gname} differs"
        assert torch.equal(grads["dS0"][s], own["dS0"][0]), f"sequence {s}: dS0 differs"
