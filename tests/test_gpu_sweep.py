"""Randomised parity sweep against the oracle, seeded: the forward (fixed-length
and packed variable-length batches), the backward and the several-token decode,
over random shapes (T up to 300, empty packed sequences), chunk sizes, input
dtypes, gate layouts and gate recipes inside the supported set.  Each case is
printed before it runs."""
import numpy as np
import pytest
import torch

import oracle
from linear_attention_sequence_chunk_amd import chunk_bwd, chunk_fwd, chunk_fwd_varlen, decode_tokens, inputs
from tests.parity import TOL, assert_close

pytestmark = pytest.mark.gpu
dev = "cuda:0"


def gate_in(d, layout):
    if layout == "channel":
        return d["g"], d["g"]
    if layout == "head":
        gh = d["g"][..., 0].contiguous()
        return gh, gh[..., None].expand_as(d["g"]).contiguous()
    return None, torch.zeros_like(d["g"])


def _run_cases(rs, NCASE):
    for case in range(NCASE):
        dk, dv = int(rs.choice([64, 128])), int(rs.choice([64, 128]))
        dtype = torch.bfloat16 if rs.random() < 0.7 else torch.float32
        C = int(rs.choice([16, 32, 64, 128] if dtype == torch.bfloat16 else [16, 32, 64]))
        layout = str(rs.choice(["channel", "head", "none"], p=[0.6, 0.25, 0.15]))
        gates = str(rs.choice(["tiny", "long"])) if layout == "channel" else "tiny"
        B, H, T = int(rs.integers(1, 4)), int(rs.integers(1, 4)), int(rs.integers(1, 300))
        s0 = float(rs.choice([0.0, 0.01, 0.3]))
        kind = str(rs.choice(["fwd", "varlen", "bwd", "decode"], p=[0.35, 0.25, 0.25, 0.15]))
        if kind == "bwd" and C == 128:
            C = 64                                            # the backward covers C <= 64
        tag = f"case {case}: {kind} dk={dk} dv={dv} C={C} {str(dtype)[6:]} {layout}/{gates} B={B} H={H} T={T} s0={s0}"
        print(tag, flush=True)
        seed = int(rs.integers(0, 1 << 20))
        tol = TOL[dtype]
        if kind == "decode":
            Tt = int(rs.integers(1, 10))
            d = inputs.custom_prefill(seed, B, Tt, H, dk, dv, dtype, gates=gates, s0_std=s0 or 0.01)
            gi, gfull = gate_in(d, layout)
            S = d["S0"].to(dev).clone()
            o = decode_tokens(d["q"].to(dev), d["k"].to(dev), d["v"].to(dev), None if gi is None else gi.to(dev),
                              d["beta"].to(dev), S, gate_layout=layout)
            torch.cuda.synchronize()
            o_ref, S_ref = oracle.recurrent(d["q"], d["k"], d["v"], gfull, d["beta"], d["S0"])
            eo = assert_close(tag + " o", o.cpu(), o_ref, tol)
            es = assert_close(tag + " S", S.cpu(), S_ref, tol)
            print(f"   T={Tt} err o {eo:.2e} S {es:.2e}", flush=True)
            continue
        d = inputs.custom_prefill(seed, B, T, H, dk, dv, dtype, gates=gates, s0_std=s0)
        gi, gfull = gate_in(d, layout)
        S0 = d["S0"]
        if kind == "fwd":
            o, S = chunk_fwd(d["q"].to(dev), d["k"].to(dev), d["v"].to(dev), None if gi is None else gi.to(dev),
                             d["beta"].to(dev), None if S0 is None else S0.to(dev), chunk_size=C, gate_layout=layout)
            torch.cuda.synchronize()
            o_ref, S_ref = oracle.recurrent(d["q"], d["k"], d["v"], gfull, d["beta"], S0)
            eo = assert_close(tag + " o", o.cpu(), o_ref, tol)
            es = assert_close(tag + " S", S.cpu(), S_ref, tol)
            print(f"   err o {eo:.2e} S {es:.2e}", flush=True)
        elif kind == "varlen":
            # B sequences' tokens packed, cut at random points (empty sequences allowed)
            flat = lambda x: None if x is None else x.reshape((B * T,) + tuple(x.shape[2:])).contiguous()
            N = int(rs.integers(1, 6))
            cuts = np.sort(rs.integers(0, B * T + 1, N - 1))
            cu = np.concatenate([[0], cuts, [B * T]]).astype(np.int32)
            q, k, v, beta = flat(d["q"]), flat(d["k"]), flat(d["v"]), flat(d["beta"])
            gin, gf = flat(gi), flat(gfull)
            S0n = torch.tensor(rs.standard_normal((N, H, dk, dv)) * (s0 or 0.0), dtype=torch.float32)
            o, S = chunk_fwd_varlen(q.to(dev), k.to(dev), v.to(dev), None if gin is None else gin.to(dev),
                                    beta.to(dev), torch.tensor(cu).to(dev), S0n.to(dev), chunk_size=C,
                                    gate_layout=layout)
            torch.cuda.synchronize()
            worst = 0.0
            for s in range(N):
                a, b = int(cu[s]), int(cu[s + 1])
                sl = lambda x: x[a:b][None]
                o_ref, S_ref = oracle.recurrent(sl(q), sl(k), sl(v), sl(gf), sl(beta), S0n[s:s + 1])
                if b > a:
                    worst = max(worst, assert_close(tag + f" o seq {s}", o[a:b].cpu(), o_ref[0], tol))
                worst = max(worst, assert_close(tag + f" S seq {s}", S[s].cpu(), S_ref[0], tol))
            print(f"   N={N} cu={cu.tolist()} worst err {worst:.2e}", flush=True)
        else:
            if T > 150:
                T = 150
                d = {key: (None if x is None else x[:, :T].contiguous() if x.dim() > 2 and key != "S0" else x)
                     for key, x in d.items()}
                gi, gfull = gate_in(d, layout)
            dO = torch.tensor(rs.standard_normal((B, T, H, dv)), dtype=torch.float32)
            dST = torch.tensor(rs.standard_normal((B, H, dk, dv)), dtype=torch.float32) if rs.random() < 0.5 else None
            got = chunk_bwd(d["q"].to(dev), d["k"].to(dev), d["v"].to(dev), None if gi is None else gi.to(dev),
                            d["beta"].to(dev), dO.to(dev), None if S0 is None else S0.to(dev),
                            None if dST is None else dST.to(dev), chunk_size=C, gate_layout=layout)
            torch.cuda.synchronize()
            ref = oracle.backward(d["q"], d["k"], d["v"], gfull, d["beta"], S0, dO, dST)
            btol = 1e-4 if dtype == torch.float32 else 2e-2
            errs = []
            for n in ("dq", "dk", "dv", "dbeta", "dS0", "dg"):
                if n == "dg":
                    if layout == "none":
                        assert got["dg"] is None
                        continue
                    want = ref["dg"].sum(-1) if layout == "head" else ref["dg"]
                else:
                    want = ref[n]
                errs.append(assert_close(tag + " " + n, got[n].cpu(), want, btol))
            print(f"   T={T} dST={'yes' if dST is not None else 'no'} worst err {max(errs):.2e}", flush=True)


@pytest.mark.parametrize("seed", [11, 12, 13, 14])
def test_random_cases(seed):
    _run_cases(np.random.default_rng(seed), 30)
