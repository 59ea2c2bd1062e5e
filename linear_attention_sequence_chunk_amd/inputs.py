"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module holds input recipes only (random draws, normalisation of the draws,
dtype casts); none of the method's arithmetic.  Both the GPU path and the CPU
oracle consume what it returns.

Random stream for a tensor slice: numpy PCG64 seeded with
``SeedSequence([0x4B4441, config_id, tensor_id, block])``; ``block`` is the
4096-token block index for prefill tensors and the step index for decode, so
any block can be regenerated alone.

Workloads (token counts and distributions follow the five workload descriptions
of the build's target; "N(0, s)" means standard deviation s):

 1 tiny    B=1 H=2  T=256     d=64  C=64   fp32 q,k,v
 2 mid     B=4 H=16 T=8192    d=128 C=64   bf16 q,k,v; gate sweeps channel / none / scalar
 3 long    B=1 H=32 T=65536   d=128 C=128  bf16; ~10% fast channels per head
 4 decode  N=256 H=32         d=128        bf16; 1000 single-token steps
 5 1m      B=1 H=16 T=1048576 d=128 C=64   bf16; 64 recurring address keys per 4096 tokens

Common recipes: q, k = L2-normalise(N(0,1)) per (b,t,h) vector in fp64;
v ~ N(0,1); beta = sigmoid(N(0,1)) per (b,t,h); "tiny" gates
g = -softplus(N(0,1) + 2) per (b,t,h,channel).
"""
from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

MAGIC = 0x4B4441
BLOCK = 4096
TENSOR_IDS = {"q": 1, "k": 2, "v": 3, "beta": 4, "g": 5, "S0": 6,
              "addr": 7, "chan_class": 8, "scalar_gate": 9}


@dataclasses.dataclass(frozen=True)
class Workload:
    cfg_id: int
    name: str
    B: int
    T: int
    H: int
    dk: int
    dv: int
    C: int
    dtype: str          # storage dtype of q, k, v: "f32" or "bf16"
    gates: str          # "tiny", "long", "none", "scalar"
    keys: str = "normal"  # "normal" or "address"
    S0: str = "zero"    # "zero" or "normal0.01"
    steps: int = 0      # decode steps (decode workload only)

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == "f32" else torch.bfloat16

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


WORKLOADS = {
    "tiny": Workload(1, "tiny", 1, 256, 2, 64, 64, 64, "f32", "tiny"),
    "mid": Workload(2, "mid", 4, 8192, 16, 128, 128, 64, "bf16", "tiny"),
    "long": Workload(3, "long", 1, 65536, 32, 128, 128, 128, "bf16", "long", S0="normal0.01"),
    "decode": Workload(4, "decode", 256, 1, 32, 128, 128, 1, "bf16", "tiny",
                       S0="normal0.01", steps=1000),
    "1m": Workload(5, "1m", 1, 1 << 20, 16, 128, 128, 64, "bf16", "long", keys="address"),
}


def rng(cfg_id: int, tensor: str, block: int) -> np.random.Generator:
    ss = np.random.SeedSequence([MAGIC, int(cfg_id), TENSOR_IDS[tensor], int(block)])
    return np.random.Generator(np.random.PCG64(ss))


def _normalize(x: np.ndarray) -> np.ndarray:
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def _sigmoid(x: np.ndarray) -> np.ndarray:
    return 1.0 / (1.0 + np.exp(-x))


def _neg_softplus(x: np.ndarray) -> np.ndarray:
    return -np.logaddexp(0.0, x)


def _threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def _store(x64: np.ndarray, dtype) -> torch.Tensor:
    """fp64 draw -> fp32 (round to nearest) -> storage dtype (torch, RNE)."""
    t = torch.from_numpy(np.ascontiguousarray(x64, dtype=np.float32))
    return t if dtype == torch.float32 else t.to(dtype)


# --------------------------------------------------------------------------- prefill
def _block_ranges(t0: int, t1: int):
    b0 = t0 // BLOCK
    while b0 * BLOCK < t1:
        s, e = b0 * BLOCK, (b0 + 1) * BLOCK
        yield b0, max(s, t0), min(e, t1)
        b0 += 1


def _addresses(w: Workload) -> np.ndarray:
    """64 fixed unit address vectors per (b,h): [B,H,64,dk]."""
    return _normalize(rng(w.cfg_id, "addr", 0).standard_normal((w.B, w.H, 64, w.dk)))


def _fast_channels(w: Workload) -> np.ndarray:
    """Per (b,h,channel) class, drawn once: True = fast-forget (alpha ~ 0.5)."""
    return rng(w.cfg_id, "chan_class", 0).random((w.B, w.H, w.dk)) < 0.1


def _gen_block(w: Workload, blk: int, s: int, e: int, gates: str, heads):
    """Generate tokens [s, e) of block ``blk`` for all tensors (fp64 draws)."""
    bs = blk * BLOCK
    n = min(BLOCK, w.T - bs)            # the block's full length
    lo, hi = s - bs, e - bs
    B, H, dk, dv = w.B, w.H, w.dk, w.dv
    hs = slice(None) if heads is None else heads

    q = _normalize(rng(w.cfg_id, "q", blk).standard_normal((B, n, H, dk)))[:, lo:hi][:, :, hs]
    kraw = rng(w.cfg_id, "k", blk).standard_normal((B, n, H, dk))
    if w.keys == "address":
        A = _addresses(w)                          # [B,H,64,dk]
        pos = (bs + np.arange(n)) % BLOCK
        sel = np.nonzero(pos < 64)[0]
        if sel.size:
            kraw[:, sel] = np.transpose(A[:, :, pos[sel]], (0, 2, 1, 3)) + 0.05 * kraw[:, sel]
    k = _normalize(kraw)[:, lo:hi][:, :, hs]
    v = rng(w.cfg_id, "v", blk).standard_normal((B, n, H, dv))[:, lo:hi][:, :, hs]
    beta = _sigmoid(rng(w.cfg_id, "beta", blk).standard_normal((B, n, H)))[:, lo:hi][:, :, hs]

    if gates == "tiny":
        g = _neg_softplus(rng(w.cfg_id, "g", blk).standard_normal((B, n, H, dk)) + 2.0)
    elif gates == "long":
        u = rng(w.cfg_id, "g", blk).random((B, n, H, dk))
        fast = _fast_channels(w)[:, None]          # [B,1,H,dk]
        alpha = np.where(fast, 0.45 + 0.10 * u, 0.95 + 0.049 * u)
        g = np.log(alpha)
    elif gates == "scalar":
        gs = _neg_softplus(rng(w.cfg_id, "scalar_gate", blk).standard_normal((B, n, H)) + 2.0)
        g = np.broadcast_to(gs[..., None], (B, n, H, dk))
    elif gates == "none":
        g = np.zeros((B, n, H, dk))
    else:
        raise ValueError(gates)
    g = g[:, lo:hi][:, :, hs]
    return q, k, v, g, beta


def make_prefill(w: Workload, gates: str | None = None, t0: int = 0, t1: int | None = None,
                 heads=None, threads: int | None = None) -> dict:
    """Inputs for tokens [t0, t1) of a prefill workload as CPU torch tensors:
    q,k [B,t,H,dk] and v [B,t,H,dv] in the storage dtype; g [B,t,H,dk], beta
    [B,t,H] and S0 [B,H,dk,dv] (or None) in fp32.  ``heads`` optionally selects
    a subset (slice or index array) of heads; S0 is sliced the same way."""
    gates = gates or w.gates
    t1 = w.T if t1 is None else t1
    hsel = heads
    nh = w.H if heads is None else len(np.arange(w.H)[heads])
    Tn = t1 - t0
    sd = w.torch_dtype
    out = {
        "q": torch.empty((w.B, Tn, nh, w.dk), dtype=sd),
        "k": torch.empty((w.B, Tn, nh, w.dk), dtype=sd),
        "v": torch.empty((w.B, Tn, nh, w.dv), dtype=sd),
        "g": torch.empty((w.B, Tn, nh, w.dk), dtype=torch.float32),
        "beta": torch.empty((w.B, Tn, nh), dtype=torch.float32),
    }

    def job(args):
        blk, s, e = args
        q, k, v, g, beta = _gen_block(w, blk, s, e, gates, hsel)
        a, b = s - t0, e - t0
        out["q"][:, a:b] = _store(q, sd)
        out["k"][:, a:b] = _store(k, sd)
        out["v"][:, a:b] = _store(v, sd)
        out["g"][:, a:b] = _store(g, torch.float32)
        out["beta"][:, a:b] = _store(beta, torch.float32)

    ranges = list(_block_ranges(t0, t1))
    nt = threads or _threads()
    if nt > 1 and len(ranges) > 1:
        with ThreadPoolExecutor(nt) as ex:
            list(ex.map(job, ranges))
    else:
        for r in ranges:
            job(r)
    out["S0"] = make_state(w, heads=hsel)
    return out


def make_state(w: Workload, heads=None):
    """Initial state [B,H,dk,dv] fp32 per the workload's recipe (None = zeros)."""
    if w.S0 == "zero":
        return None
    S0 = 0.01 * rng(w.cfg_id, "S0", 0).standard_normal((w.B, w.H, w.dk, w.dv))
    if heads is not None:
        S0 = S0[:, heads]
    return _store(S0, torch.float32)


# --------------------------------------------------------------------------- decode
def make_decode_step(w: Workload, step: int, seqs=None, heads=None) -> dict:
    """One decode step's inputs: q,k [N,H,dk], v [N,H,dv] in the storage dtype;
    g [N,H,dk], beta [N,H] fp32.  Optional subsets of sequences / heads."""
    N, H, dk, dv = w.B, w.H, w.dk, w.dv
    q = _normalize(rng(w.cfg_id, "q", step).standard_normal((N, H, dk)))
    k = _normalize(rng(w.cfg_id, "k", step).standard_normal((N, H, dk)))
    v = rng(w.cfg_id, "v", step).standard_normal((N, H, dv))
    beta = _sigmoid(rng(w.cfg_id, "beta", step).standard_normal((N, H)))
    g = _neg_softplus(rng(w.cfg_id, "g", step).standard_normal((N, H, dk)) + 2.0)
    sel = (slice(None) if seqs is None else seqs, slice(None) if heads is None else heads)
    sd = w.torch_dtype
    return {"q": _store(q[sel], sd), "k": _store(k[sel], sd), "v": _store(v[sel], sd),
            "g": _store(g[sel], torch.float32), "beta": _store(beta[sel], torch.float32)}


def make_decode_steps(w: Workload, steps: int, seqs=None, heads=None,
                      threads: int | None = None) -> dict:
    """``steps`` consecutive decode steps stacked on a leading axis."""
    nt = threads or _threads()
    with ThreadPoolExecutor(nt) as ex:
        parts = list(ex.map(lambda s: make_decode_step(w, s, seqs, heads), range(steps)))
    return {key: torch.stack([p[key] for p in parts]) for key in parts[0]}


def decode_state(w: Workload, seqs=None, heads=None):
    """Decode initial state [N,H,dk,dv] fp32."""
    S0 = 0.01 * rng(w.cfg_id, "S0", 0).standard_normal((w.B, w.H, w.dk, w.dv))
    if seqs is not None:
        S0 = S0[seqs]
    if heads is not None:
        S0 = S0[:, heads]
    return _store(S0, torch.float32)


def custom_prefill(seed: int, B: int, T: int, H: int, dk: int, dv: int, dtype=torch.float32,
                   gates: str = "tiny", s0_std: float = 0.0) -> dict:
    """Small ad-hoc inputs (edge cases): same recipes, own seed space
    (config id 1000 + seed), any shape."""
    w = Workload(1000 + seed, "custom", B, T, H, dk, dv, 64,
                 "f32" if dtype == torch.float32 else "bf16", gates,
                 S0="zero" if s0_std == 0 else "normal0.01")
    out = make_prefill(w, threads=1)
    if s0_std and s0_std != 0.01:
        out["S0"] = out["S0"] * (s0_std / 0.01)
    return out
