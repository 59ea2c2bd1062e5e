"""kda_chunk_fwd_noalloc (the entry point that allocates nothing: its workspace
is the library's static device array) on the GPU, called through the C ABI.

Two calls in a row, the first close to the array's size, the second smaller:
each must equal kda_chunk_fwd_ex on the same inputs (with its own workspace),
bitwise, and the fp64 oracle at the parity bar.  The second call reuses the
array the first one filled."""
import pytest
import torch

import oracle
from linear_attention_sequence_chunk_amd import _lib, chunk_fwd, inputs
from tests.parity import TOL, assert_close, cuda

pytestmark = pytest.mark.gpu


def _largest_T(B, H, dk, dv, C, T_hi):
    """The longest sequence (a multiple of 100 tokens, up to T_hi) whose
    workspace fits the static array."""
    L = _lib.lib()
    code = _lib.BF16
    T = T_hi
    while T > 100 and L.kda_chunk_fwd_workspace_bytes(B, T, H, dk, dv, code, C) > _lib.NOALLOC_WORKSPACE_MAX:
        T -= 100
    return T


def _noalloc(d, C, out_dtype, gate_layout):
    """The C entry point, with outputs allocated here (by torch, the caller)."""
    B, T, H, dk = d["q"].shape
    dv = d["v"].shape[-1]
    o = torch.empty((B, T, H, dv), dtype=out_dtype, device="cuda:0")
    S = torch.empty((B, H, dk, dv), dtype=torch.float32, device="cuda:0")
    p = lambda x: None if x is None else x.data_ptr()
    st = _lib.lib().kda_chunk_fwd_noalloc(
        p(d["q"]), p(d["k"]), p(d["v"]), p(d["g"]), p(d["beta"]), p(d["S0"]), p(o), p(S), B, T, H, dk, dv,
        _lib.BF16 if d["q"].dtype == torch.bfloat16 else _lib.F32,
        _lib.BF16 if out_dtype == torch.bfloat16 else _lib.F32,
        torch.cuda.current_stream().cuda_stream, C, _lib.GATE[gate_layout])
    assert st == 0, _lib.status_string(st)
    return o, S


def test_noalloc_two_calls_match_the_workspace_entry_point():
    H, dk, dv, C = 16, 128, 128, 64
    T1 = _largest_T(1, H, dk, dv, C, 8000)
    calls = [dict(B=1, T=T1, H=H, dtype=torch.bfloat16, out=torch.bfloat16, gates="tiny", layout="channel"),
             dict(B=2, T=300, H=3, dtype=torch.bfloat16, out=torch.float32, gates="scalar", layout="head")]
    for i, c in enumerate(calls):
        print(f"no-alloc call {i}: B={c['B']} T={c['T']} H={c['H']} gates={c['layout']}", flush=True)
        h = inputs.custom_prefill(71 + i, c["B"], c["T"], c["H"], dk, dv, dtype=c["dtype"], gates=c["gates"],
                                  s0_std=0.02)
        if c["layout"] == "head":
            h["g"] = h["g"][..., 0].contiguous()
        d = cuda(h)
        o, S = _noalloc(d, C, c["out"], c["layout"])
        o_ref, S_ref = chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["S0"], chunk_size=C,
                                 out_dtype=c["out"], gate_layout=c["layout"])
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref) and torch.equal(S, S_ref), f"call {i}: differs from kda_chunk_fwd_ex"
        g64 = h["g"] if c["layout"] == "channel" else h["g"][..., None].expand(h["q"].shape).contiguous()
        oo, SS = oracle.recurrent(h["q"], h["k"], h["v"], g64, h["beta"], h["S0"])
        eo = assert_close(f"call {i} o", o.cpu(), oo, TOL[torch.bfloat16])
        es = assert_close(f"call {i} S", S.cpu(), SS, TOL[torch.bfloat16])
        print(f"  max err o {eo:.2e} S {es:.2e}", flush=True)
