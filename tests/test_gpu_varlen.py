"""Packed variable-length batches (kda_chunk_fwd_varlen) on the GPU.

Each sequence of the packed call must equal, bitwise, a fixed-length
kda_chunk_fwd call on that sequence alone, and the fp64 oracle to the parity
bar.  Lengths cover the edge cases: empty sequences, one token, chunk
boundaries +- 1, several chunks."""
import numpy as np
import pytest
import torch

import oracle
from linear_attention_sequence_chunk_amd import chunk_fwd, chunk_fwd_varlen, inputs
from tests.parity import TOL, assert_close

pytestmark = pytest.mark.gpu

CONFIGS = [(128, 128, 64, torch.bfloat16), (128, 64, 64, torch.bfloat16), (64, 64, 32, torch.float32),
           (128, 128, 128, torch.bfloat16), (64, 128, 16, torch.float32)]


def _packed(lengths, H, dk, dv, dtype, gates, s0_std, seed):
    seqs = []
    for i, L in enumerate(lengths):
        d = inputs.custom_prefill(seed * 100 + i, 1, max(L, 1), H, dk, dv, dtype=dtype, gates=gates,
                                  s0_std=s0_std)
        seqs.append({k: (v[:, :L] if k not in ("S0",) and v is not None else v) for k, v in d.items()})
    cat = lambda key: torch.cat([s[key][0] for s in seqs], dim=0)     # [T, H, ...]
    S0 = torch.cat([s["S0"] for s in seqs], dim=0) if s0_std else None
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lengths)]), dtype=torch.int32)
    return seqs, {k: cat(k) for k in ("q", "k", "v", "g", "beta")}, S0, cu


def _run_and_check(lengths, H, dk, dv, C, dtype, layout="channel", s0_std=0.05, seed=1, oracle_every=1):
    gates = {"channel": "tiny", "head": "scalar", "none": "none"}[layout]
    seqs, p, S0, cu = _packed(lengths, H, dk, dv, dtype, gates, s0_std, seed)
    dev = "cuda:0"
    gsel = lambda g: None if layout == "none" else (g[..., 0].contiguous() if layout == "head" else g)
    o, S = chunk_fwd_varlen(p["q"].to(dev), p["k"].to(dev), p["v"].to(dev), None if gsel(p["g"]) is None
                            else gsel(p["g"]).to(dev), p["beta"].to(dev), cu.to(dev),
                            None if S0 is None else S0.to(dev), chunk_size=C, gate_layout=layout)
    torch.cuda.synchronize()
    o, S = o.cpu(), S.cpu()
    offs = cu.tolist()
    for i, (L, d) in enumerate(zip(lengths, seqs)):
        s0 = None if S0 is None else S0[i:i + 1].to(dev)
        gi = gsel(d["g"])
        oi, Si = chunk_fwd(d["q"].to(dev), d["k"].to(dev), d["v"].to(dev), None if gi is None else gi.to(dev),
                           d["beta"].to(dev), s0, chunk_size=C, gate_layout=layout)
        torch.cuda.synchronize()
        seg = o[offs[i]:offs[i + 1]]
        if L:
            assert torch.equal(seg, oi[0].cpu()), f"sequence {i} (length {L}): o differs from its own call"
        assert torch.equal(S[i], Si[0].cpu()), f"sequence {i} (length {L}): state differs from its own call"
        if i % oracle_every == 0:
            g_ref = torch.zeros_like(d["g"]) if layout == "none" else d["g"]
            o_ref, S_ref = oracle.recurrent(d["q"], d["k"], d["v"], g_ref, d["beta"],
                                            None if S0 is None else S0[i:i + 1])
            if L:
                assert_close(f"seq {i} o", seg[None], o_ref, TOL[dtype])
            assert_close(f"seq {i} S", S[i:i + 1], S_ref, TOL[dtype])


@pytest.mark.parametrize("dk,dv,C,dtype", CONFIGS)
def test_varlen_edge_lengths(dk, dv, C, dtype):
    lengths = [0, 1, C - 1, C, C + 1, 3 * C + 5, 7, 0, 2 * C]
    print(f"varlen dk={dk} dv={dv} C={C} {dtype} lengths={lengths}", flush=True)
    _run_and_check(lengths, 3, dk, dv, C, dtype)


@pytest.mark.parametrize("layout", ["head", "none"])
def test_varlen_gate_layouts(layout):
    _run_and_check([5, 64, 0, 130, 1], 2, 128, 128, 64, torch.bfloat16, layout=layout, seed=2)


def test_varlen_many_sequences():
    """2500 sequences (the chunk-offset scan spans three 1024-sequence blocks)."""
    rs = np.random.default_rng(3)
    lengths = [int(x) for x in rs.integers(0, 90, 2500)]
    print(f"varlen many: {len(lengths)} sequences, {sum(lengths)} tokens", flush=True)
    _run_and_check(lengths, 2, 128, 128, 64, torch.bfloat16, s0_std=0.0, seed=4, oracle_every=97)


def test_varlen_no_states_and_empty():
    """No initial state (zeros), all-empty batch: final states are zero / copied."""
    _run_and_check([0, 0, 0], 2, 128, 128, 64, torch.bfloat16, s0_std=0.05, seed=5)
    _run_and_check([10, 0, 70], 2, 128, 128, 64, torch.bfloat16, s0_std=0.0, seed=6)


def test_varlen_bench_batch_full():
    """The packed batch bench.py times: the mid workload's batch rows 0 and 1
    (16384 tokens, 16 heads) cut into sequences of 64..2047 tokens by the same
    seeded draw; every output and final state of every sequence against the
    oracle."""
    w = inputs.WORKLOADS["mid"]
    d = inputs.make_prefill(w)
    T = 2 * w.T
    rs = np.random.default_rng(11)
    cuts = [0]
    while cuts[-1] < T:
        cuts.append(min(T, cuts[-1] + int(rs.integers(64, 2048))))
    pk = {key: d[key][:2].reshape((T,) + tuple(d[key].shape[2:])).contiguous()
          for key in ("q", "k", "v", "g", "beta")}
    cu = torch.tensor(cuts, dtype=torch.int32)
    print(f"varlen bench batch: {len(cuts) - 1} sequences, {T} tokens, {w.H} heads", flush=True)
    o, S = chunk_fwd_varlen(*(pk[key].cuda() for key in ("q", "k", "v", "g", "beta")), cu.cuda(),
                            chunk_size=w.C)
    torch.cuda.synchronize()
    o, S = o.cpu(), S.cpu()
    worst_o = worst_s = 0.0
    for i in range(len(cuts) - 1):
        a, b = cuts[i], cuts[i + 1]
        sl = lambda x: x[a:b][None]
        o_ref, S_ref = oracle.recurrent(sl(pk["q"]), sl(pk["k"]), sl(pk["v"]), sl(pk["g"]), sl(pk["beta"]), None)
        worst_o = max(worst_o, assert_close(f"seq {i} o", o[a:b][None], o_ref, TOL[torch.bfloat16]))
        worst_s = max(worst_s, assert_close(f"seq {i} S", S[i:i + 1], S_ref, TOL[torch.bfloat16]))
    print(f"  max err o {worst_o:.2e}  S {worst_s:.2e}", flush=True)
