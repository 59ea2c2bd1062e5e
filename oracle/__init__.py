"""fp64 CPU oracle for the KDA / gated delta-rule state update.

TEST INFRASTRUCTURE ONLY: only tests/, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` import this package.  It shares no code
with the GPU library and never imports it.

Functions and the passages they follow (pages cited by title and section):

``recurrent``       C implementation (kda_oracle.c): the per-token update in the
                    order decay -> read -> error -> write of section 八 of
                    "我终于看懂了 KDA…", the delta rule of its section 六 and of the
                    delta-rule paragraph of "一个KimiK3装下22580个GPT-2…", the
                    per-channel gate of that essay's Kimi Linear paragraph.
``recurrent_np``    the same definition in numpy, vectorised over (b,h).
``chunked_np``      the chunkwise form: chunks of C tokens, masked attention
                    inside a chunk (score first) and a state recurrence between
                    chunks (state first), C=1 being the recurrence and C=T full
                    masked attention (chunk paragraph of the KimiK3 essay;
                    section 十六 of the explainer), with the chunk's rank-1
                    updates folded into matrix form (section 十七, WY / DPLR).
                    Uses direct pairwise decays exp(G_r - G_i), no factoring.
``recurrent_exact`` exact rational arithmetic (fractions) of the definition,
                    taking alpha directly, for tiny sizes.
``backward``        C implementation: the fp64 adjoint of ``recurrent`` (reverse
                    sweep over the tokens of the same per-token update), giving
                    the gradients of sum(dO * o) + sum(dST * S_T) for training
                    the chunkwise form (sections 十六 and 十七 of the explainer).
``l2_normalize``    the steps that produce q, k and g in the method's workloads
``gate_softplus``   (inputs of the path, not the path): each [d] row divided by
                    its Euclidean norm, and the log-gate -softplus(a) =
                    -log(1 + e^a); the oracle side of the fused pre-processing.
``l2_normalize_vjp``  their vector-Jacobian products, written out from the
``gate_softplus_vjp`` derivatives of those definitions: (I - y y^T)/|x| for
                    y = x/|x|, and -sigmoid(a); the oracle side of the backward
                    pass through the fused pre-processing.

Parity pins: every function here is pinned by tests/test_oracle_pins.py to
closed forms, special cases and library routines (least squares, finite
differences, exact rationals); none is "parity unpinned".
"""
from __future__ import annotations

import ctypes
import os
from fractions import Fraction

import numpy as np

from . import build as _build

_LIB = None


def _lib():
    global _LIB
    if _LIB is None:
        path = _build.ensure_built()
        lib = ctypes.CDLL(path)
        dp = ctypes.POINTER(ctypes.c_double)
        lib.kda_oracle_recurrent.argtypes = [ctypes.c_int] * 5 + [dp] * 8 + [
            ctypes.c_int, dp, ctypes.c_int]
        lib.kda_oracle_recurrent.restype = None
        lib.kda_oracle_last_threads.argtypes = []
        lib.kda_oracle_last_threads.restype = ctypes.c_int
        lib.kda_oracle_backward.argtypes = [ctypes.c_int] * 5 + [dp] * 14 + [ctypes.c_int, ctypes.c_int]
        lib.kda_oracle_backward.restype = None
        _LIB = lib
    return _LIB


def to_f64(x):
    """Exact upcast of a stored input (numpy or torch, any float dtype) to fp64."""
    if x is None:
        return None
    try:
        import torch  # plumbing only: bf16 storage lives in torch tensors
        if isinstance(x, torch.Tensor):
            return x.detach().to("cpu", torch.float64).contiguous().numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(a):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def recurrent(q, k, v, g, beta, S0=None, delta=True, dump_u=False, nthreads=0):
    """Sequential fp64 recurrence.  Shapes q,k,g [B,T,H,dk], v [B,T,H,dv],
    beta [B,T,H], S0 [B,H,dk,dv] or None.  Returns (o, S_T) or (o, S_T, u)."""
    q, k, v, g, beta, S0 = (to_f64(a) for a in (q, k, v, g, beta, S0))
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    assert k.shape == (B, T, H, dk) and g.shape == (B, T, H, dk)
    assert v.shape == (B, T, H, dv) and beta.shape == (B, T, H)
    if S0 is not None:
        assert S0.shape == (B, H, dk, dv)
    o = np.empty((B, T, H, dv), np.float64)
    ST = np.empty((B, H, dk, dv), np.float64)
    u = np.empty((B, T, H, dv), np.float64) if dump_u else None
    _lib().kda_oracle_recurrent(B, T, H, dk, dv, _ptr(q), _ptr(k), _ptr(v), _ptr(g),
                                _ptr(beta), _ptr(S0), _ptr(o), _ptr(ST),
                                1 if delta else 0, _ptr(u), int(nthreads))
    return (o, ST, u) if dump_u else (o, ST)


def backward(q, k, v, g, beta, S0=None, dO=None, dST=None, seg=64, nthreads=0):
    """fp64 adjoint of ``recurrent`` for L = sum(dO * o) + sum(dST * S_T).
    Returns dict(dq, dk, dv, dg, dbeta, dS0) as fp64 arrays."""
    q, k, v, g, beta, S0, dO, dST = (to_f64(a) for a in (q, k, v, g, beta, S0, dO, dST))
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    out = {"dq": np.zeros((B, T, H, dk)), "dk": np.zeros((B, T, H, dk)), "dv": np.zeros((B, T, H, dv)),
           "dg": np.zeros((B, T, H, dk)), "dbeta": np.zeros((B, T, H)), "dS0": np.zeros((B, H, dk, dv))}
    _lib().kda_oracle_backward(B, T, H, dk, dv, _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(S0),
                               _ptr(dO), _ptr(dST), _ptr(out["dq"]), _ptr(out["dk"]), _ptr(out["dv"]),
                               _ptr(out["dg"]), _ptr(out["dbeta"]), _ptr(out["dS0"]), int(seg), int(nthreads))
    return out


def last_threads() -> int:
    return int(_lib().kda_oracle_last_threads())


def recurrent_np(q, k, v, g, beta, S0=None, delta=True):
    """numpy twin of ``recurrent`` (same definition, vectorised over b,h)."""
    q, k, v, g, beta, S0 = (to_f64(a) for a in (q, k, v, g, beta, S0))
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    S = np.zeros((B, H, dk, dv)) if S0 is None else S0.copy()
    o = np.empty((B, T, H, dv))
    for t in range(T):
        S = np.exp(g[:, t])[..., None] * S                       # decay rows
        r = np.einsum("bhc,bhcj->bhj", k[:, t], S) if delta else 0.0  # read
        u = beta[:, t, :, None] * (v[:, t] - r)                   # error * beta
        S = S + k[:, t, :, :, None] * u[:, :, None, :]            # write
        o[:, t] = np.einsum("bhc,bhcj->bhj", q[:, t], S)          # output
    return o, S


def chunked_np(q, k, v, g, beta, S0=None, C=64):
    """Chunkwise-parallel form in fp64 for any C >= 1 and any T (the last chunk
    may be partial).  Per chunk with local positions r, i and start state S:

        G   = inclusive cumulative sum of g over the chunk (per channel)
        D   = exp(G_r - G_i) for i <= r                  (direct, no factoring)
        A   = sum_c k_r k_i D  for i < r                 (strictly lower)
        P   = sum_c q_r k_i D  for i <= r                (lower, with diagonal)
        T   = (I + Diag(beta) A)^-1
        U   = T Diag(beta) V ;  Wk = T Diag(beta) (exp(G) * K)
        W   = U - Wk S                                   (row r = u_r)
        O   = (exp(G) * Q) S + P W
        S  <- Diag(exp(G_last)) S + (exp(G_last - G) * K)^T W

    Requires finite g (the pairwise differences of -inf are undefined)."""
    q, k, v, g, beta, S0 = (to_f64(a) for a in (q, k, v, g, beta, S0))
    assert np.all(np.isfinite(g)), "chunked_np needs finite log-gates"
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    o = np.empty((B, T, H, dv))
    ST = np.empty((B, H, dk, dv))
    for b in range(B):
        for h in range(H):
            S = np.zeros((dk, dv)) if S0 is None else S0[b, h].copy()
            for s in range(0, T, C):
                e = min(s + C, T)
                Q, K, V = q[b, s:e, h], k[b, s:e, h], v[b, s:e, h]
                bet = beta[b, s:e, h]
                G = np.cumsum(g[b, s:e, h], axis=0)
                n = e - s
                lower = np.tril(np.ones((n, n), bool))
                D = np.where(lower[:, :, None], np.exp(G[:, None, :] - G[None, :, :]), 0.0)
                A = np.einsum("rc,ic,ric->ri", K, K, D) * np.tril(np.ones((n, n)), -1)
                P = np.einsum("rc,ic,ric->ri", Q, K, D)
                Tm = np.linalg.inv(np.eye(n) + bet[:, None] * A)
                U = Tm @ (bet[:, None] * V)
                Wk = Tm @ (bet[:, None] * (np.exp(G) * K))
                W = U - Wk @ S
                o[b, s:e, h] = (np.exp(G) * Q) @ S + P @ W
                S = np.exp(G[-1])[:, None] * S + (np.exp(G[-1] - G) * K).T @ W
            ST[b, h] = S
    return o, ST


def recurrent_exact(q, k, v, alpha, beta, S0=None, delta=True):
    """Exact rational recurrence for tiny sizes.  Inputs are nested lists (or
    arrays) of numbers convertible to Fraction; alpha replaces exp(g).
    Shapes: q,k,alpha [T][dk], v [T][dv], beta [T], S0 [dk][dv].  Returns
    (o [T][dv], S [dk][dv]) as Fractions."""
    F = Fraction
    T = len(q)
    dk, dv = len(q[0]), len(v[0])
    S = [[F(0)] * dv for _ in range(dk)] if S0 is None else [[F(x) for x in row] for row in S0]
    out = []
    for t in range(T):
        a = [F(x) for x in alpha[t]]
        kt = [F(x) for x in k[t]]
        qt = [F(x) for x in q[t]]
        vt = [F(x) for x in v[t]]
        bt = F(beta[t])
        S = [[a[c] * S[c][j] for j in range(dv)] for c in range(dk)]
        r = [sum((kt[c] * S[c][j] for c in range(dk)), F(0)) if delta else F(0) for j in range(dv)]
        u = [bt * (vt[j] - r[j]) for j in range(dv)]
        S = [[S[c][j] + kt[c] * u[j] for j in range(dv)] for c in range(dk)]
        out.append([sum((qt[c] * S[c][j] for c in range(dk)), F(0)) for j in range(dv)])
    return out, S


def l2_normalize(x):
    """Each row (last axis) divided by its Euclidean norm, in fp64; a zero row
    stays zero."""
    x = to_f64(x)
    n = np.sqrt(np.sum(x * x, axis=-1, keepdims=True))
    return np.divide(x, n, out=np.zeros_like(x), where=n > 0)


def gate_softplus(a):
    """The log-gate -softplus(a) = -log(1 + e^a), in fp64 (alpha = 1/(1 + e^a))."""
    a = to_f64(a)
    return -(np.maximum(a, 0.0) + np.log1p(np.exp(-np.abs(a))))


def l2_normalize_vjp(x, dy):
    """Gradient with respect to x of sum(dy * l2_normalize(x)), in fp64.  With
    y = x/|x| the Jacobian is (I - y y^T)/|x|, so dx = (dy - y (y . dy))/|x|.  A
    zero row, where the normalisation is defined as zero, gets zero."""
    x, dy = to_f64(x), to_f64(dy)
    n = np.sqrt(np.sum(x * x, axis=-1, keepdims=True))
    y = np.divide(x, n, out=np.zeros_like(x), where=n > 0)
    inv = np.divide(1.0, n, out=np.zeros_like(n), where=n > 0)
    return (dy - y * np.sum(y * dy, axis=-1, keepdims=True)) * inv


def gate_softplus_vjp(a, dg):
    """Gradient with respect to a of sum(dg * gate_softplus(a)), in fp64: the
    derivative of -log(1 + e^a) is -1/(1 + e^-a) = -sigmoid(a)."""
    a, dg = to_f64(a), to_f64(dg)
    e = np.exp(-np.abs(a))
    sig = np.where(a >= 0, 1.0 / (1.0 + e), e / (1.0 + e))
    return -dg * sig


def lib_path() -> str:
    return os.path.abspath(_build.LIB)
