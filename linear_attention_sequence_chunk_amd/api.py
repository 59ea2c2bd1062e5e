"""Thin torch binding over the C ABI: argument checks and marshalling only.
Every step of the computation runs in the HIP kernels of libkda.so."""
from __future__ import annotations

import torch

from . import _lib

_DT = {torch.float32: _lib.F32, torch.bfloat16: _lib.BF16}


def _code(dtype) -> int:
    if dtype not in _DT:
        raise TypeError(f"unsupported dtype {dtype}; use float32 or bfloat16")
    return _DT[dtype]


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(stream, device) -> int:
    """The raw HIP stream: the given one, else torch's current stream on the
    tensors' device."""
    s = torch.cuda.current_stream(device) if stream is None else stream
    return s.cuda_stream


def _check_tensor(name, t, shape, dtype, device):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def workspace_bytes(B, T, H, dk, dv, in_dtype, chunk_size) -> int:
    return int(_lib.lib().kda_chunk_fwd_workspace_bytes(B, T, H, dk, dv, _code(in_dtype), chunk_size))


def _gate(layout) -> int:
    if layout not in _lib.GATE:
        raise ValueError(f"gate_layout must be one of {sorted(_lib.GATE)}")
    return _lib.GATE[layout]


def _check_gate(g, layout, lead, dk, dev, allow_bf16=False):
    """g is [*lead, dk] per channel, [*lead] per head, None (or ignored) without
    gates; fp32, or bf16 where the call takes pre-processing flags."""
    if layout == "none":
        return
    dt = g.dtype if allow_bf16 and isinstance(g, torch.Tensor) and g.dtype == torch.bfloat16 else torch.float32
    _check_tensor("g", g, tuple(lead) + ((dk,) if layout == "channel" else ()), dt, dev)


def _pre_flags(qk_l2norm, gate_act, g, layout) -> int:
    """kda_pre_flags_t for the binding's keywords: q/k normalised in the kernels,
    the gate given as a pre-activation ("softplus": log-gate = -softplus(g)), and
    a bf16 gate tensor."""
    if gate_act not in (None, "softplus"):
        raise ValueError('gate_act must be None or "softplus"')
    f = _lib.PRE_QK_L2NORM if qk_l2norm else 0
    if layout != "none":
        if gate_act == "softplus":
            f |= _lib.PRE_GATE_SOFTPLUS
        if isinstance(g, torch.Tensor) and g.dtype == torch.bfloat16:
            f |= _lib.PRE_GATE_BF16
    return f


def _prep_chunk(q, k, v, g, beta, initial_state, chunk_size, out_dtype, final_state, workspace,
                gate_layout="channel", allow_bf16_gate=False):
    _gate(gate_layout)
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("inputs must be on a GPU")
    _check_tensor("q", q, (B, T, H, dk), q.dtype, dev)
    _check_tensor("k", k, (B, T, H, dk), q.dtype, dev)
    _check_tensor("v", v, (B, T, H, dv), q.dtype, dev)
    _check_gate(g, gate_layout, (B, T, H), dk, dev, allow_bf16_gate)
    _check_tensor("beta", beta, (B, T, H), torch.float32, dev)
    if initial_state is not None:
        _check_tensor("initial_state", initial_state, (B, H, dk, dv), torch.float32, dev)
    out_dtype = q.dtype if out_dtype is None else out_dtype
    o = torch.empty((B, T, H, dv), dtype=out_dtype, device=dev)
    if final_state is None:
        final_state = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)
    else:
        _check_tensor("final_state", final_state, (B, H, dk, dv), torch.float32, dev)
    nbytes = workspace_bytes(B, T, H, dk, dv, q.dtype, chunk_size)
    if workspace is None:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)
    return (B, T, H, dk, dv, out_dtype, o, final_state, workspace)


def _call_chunk(fn_name, q, k, v, g, beta, initial_state, o, final_state, B, T, H, dk, dv,
                out_dtype, workspace, chunk_size, stream, gate_layout="channel", pre=0):
    args = [_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(initial_state), _ptr(o),
            _ptr(final_state), B, T, H, dk, dv, _code(q.dtype), _code(out_dtype),
            _ptr(workspace), workspace.numel(), _stream(stream, q.device), chunk_size]
    if pre and fn_name in ("kda_chunk_fwd", "kda_chunk_intra"):
        fn_name, args = fn_name + "_pre", args + [_gate(gate_layout), pre]
    elif gate_layout != "channel" and fn_name in ("kda_chunk_fwd", "kda_chunk_intra"):
        fn_name, args = fn_name + "_ex", args + [_gate(gate_layout)]
    st = getattr(_lib.lib(), fn_name)(*args)
    _lib.check(st, fn_name)


def chunk_fwd(q, k, v, g, beta, initial_state=None, chunk_size=64, out_dtype=None,
              final_state=None, workspace=None, stream=None, gate_layout="channel",
              qk_l2norm=False, gate_act=None):
    """Chunkwise KDA forward (kda_chunk_fwd / _ex / _pre).  q,k [B,T,H,dk],
    v [B,T,H,dv] in fp32 or bf16; beta [B,T,H] fp32; g fp32 [B,T,H,dk]
    (gate_layout "channel"), [B,T,H] ("head") or None ("none"); initial_state
    [B,H,dk,dv] fp32 or None.  Returns (o [B,T,H,dv], final_state [B,H,dk,dv] fp32).
    ``final_state`` may be given (e.g. the initial_state tensor, for in place).
    Fused pre-processing: ``qk_l2norm`` normalises q and k rows in the kernels;
    ``gate_act="softplus"`` takes g as a pre-activation (log-gate -softplus(g));
    g may then also be bf16."""
    pre = _pre_flags(qk_l2norm, gate_act, g, gate_layout)
    B, T, H, dk, dv, out_dtype, o, fs, ws = _prep_chunk(q, k, v, g, beta, initial_state, chunk_size,
                                                        out_dtype, final_state, workspace, gate_layout,
                                                        allow_bf16_gate=True)
    _call_chunk("kda_chunk_fwd", q, k, v, g, beta, initial_state, o, fs, B, T, H, dk, dv,
                out_dtype, ws, chunk_size, stream, gate_layout, pre)
    return o, fs


def chunk_fwd_noalloc(q, k, v, g, beta, initial_state=None, chunk_size=64, out_dtype=None, o=None,
                      final_state=None, stream=None, gate_layout="channel"):
    """kda_chunk_fwd_noalloc: chunk_fwd with the library's static workspace (no
    workspace argument; sizes whose workspace exceeds NOALLOC_WORKSPACE_MAX
    raise).  ``o`` and ``final_state`` may be given so that nothing is allocated
    here either.  Returns (o, final_state)."""
    _gate(gate_layout)
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("inputs must be on a GPU")
    _check_tensor("k", k, (B, T, H, dk), q.dtype, dev)
    _check_tensor("v", v, (B, T, H, dv), q.dtype, dev)
    _check_gate(g, gate_layout, (B, T, H), dk, dev)
    _check_tensor("beta", beta, (B, T, H), torch.float32, dev)
    if initial_state is not None:
        _check_tensor("initial_state", initial_state, (B, H, dk, dv), torch.float32, dev)
    out_dtype = q.dtype if out_dtype is None else out_dtype
    if o is None:
        o = torch.empty((B, T, H, dv), dtype=out_dtype, device=dev)
    else:
        _check_tensor("o", o, (B, T, H, dv), out_dtype, dev)
    if final_state is None:
        final_state = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)
    else:
        _check_tensor("final_state", final_state, (B, H, dk, dv), torch.float32, dev)
    st = _lib.lib().kda_chunk_fwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(initial_state),
                                          _ptr(o), _ptr(final_state), B, T, H, dk, dv, _code(q.dtype),
                                          _code(out_dtype), _stream(stream, dev), chunk_size, _gate(gate_layout))
    _lib.check(st, "kda_chunk_fwd_noalloc")
    return o, final_state


def chunk_fwd_varlen(q, k, v, g, beta, cu_seqlens, initial_state=None, chunk_size=64, out_dtype=None,
                     final_state=None, workspace=None, stream=None, gate_layout="channel"):
    """Packed variable-length batch (kda_chunk_fwd_varlen).  q,k [T,H,dk],
    v [T,H,dv], beta [T,H]: N sequences one after another, sequence s being
    tokens cu_seqlens[s]..cu_seqlens[s+1]-1 (cu_seqlens: int32 [N+1] on the same
    GPU); g fp32 [T,H,dk] ("channel"), [T,H] ("head") or None ("none");
    initial_state [N,H,dk,dv] fp32 or None.  Returns (o [T,H,dv], final_state
    [N,H,dk,dv] fp32)."""
    _gate(gate_layout)
    T, H, dk = q.shape
    dv = v.shape[-1]
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("inputs must be on a GPU")
    N = cu_seqlens.numel() - 1
    if N < 0:
        raise ValueError("cu_seqlens needs at least one entry")
    _check_tensor("cu_seqlens", cu_seqlens, (N + 1,), torch.int32, dev)
    _check_tensor("k", k, (T, H, dk), q.dtype, dev)
    _check_tensor("v", v, (T, H, dv), q.dtype, dev)
    _check_gate(g, gate_layout, (T, H), dk, dev)
    _check_tensor("beta", beta, (T, H), torch.float32, dev)
    if initial_state is not None:
        _check_tensor("initial_state", initial_state, (N, H, dk, dv), torch.float32, dev)
    out_dtype = q.dtype if out_dtype is None else out_dtype
    o = torch.empty((T, H, dv), dtype=out_dtype, device=dev)
    if final_state is None:
        final_state = torch.empty((N, H, dk, dv), dtype=torch.float32, device=dev)
    else:
        _check_tensor("final_state", final_state, (N, H, dk, dv), torch.float32, dev)
    L = _lib.lib()
    nbytes = int(L.kda_chunk_varlen_workspace_bytes(N, T, H, dk, dv, _code(q.dtype), chunk_size))
    if workspace is None:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)
    st = L.kda_chunk_fwd_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(initial_state), _ptr(o),
                                _ptr(final_state), _ptr(cu_seqlens), N, T, H, dk, dv, _code(q.dtype),
                                _code(out_dtype), _ptr(workspace), workspace.numel(), _stream(stream, dev),
                                chunk_size, _gate(gate_layout))
    _lib.check(st, "kda_chunk_fwd_varlen")
    return o, final_state


def chunk_bwd(q, k, v, g, beta, dO, initial_state=None, dST=None, chunk_size=64, gate_layout="channel",
              workspace=None, stream=None, qk_l2norm=False, gate_act=None):
    """Backward pass (kda_chunk_bwd): gradients of L = sum(dO * o) + sum(dST * S_T)
    for the forward chunk_fwd(q, k, v, g, beta, initial_state, gate_layout=...).
    dO [B,T,H,dv] fp32, dST [B,H,dk,dv] fp32 or None.  Returns a dict of fp32
    tensors dq, dk, dv, dg (None without gates), dbeta, dS0.  With qk_l2norm or
    gate_act="softplus" (or a bf16 g), the forward is the one with those
    keywords (kda_chunk_bwd_pre) and dq, dk, dg are the gradients of the raw
    q, k and gate tensor."""
    _gate(gate_layout)
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("inputs must be on a GPU")
    pre = _pre_flags(qk_l2norm, gate_act, g, gate_layout)
    _check_tensor("k", k, (B, T, H, dk), q.dtype, dev)
    _check_tensor("v", v, (B, T, H, dv), q.dtype, dev)
    _check_gate(g, gate_layout, (B, T, H), dk, dev, allow_bf16=True)
    _check_tensor("beta", beta, (B, T, H), torch.float32, dev)
    _check_tensor("dO", dO, (B, T, H, dv), torch.float32, dev)
    if initial_state is not None:
        _check_tensor("initial_state", initial_state, (B, H, dk, dv), torch.float32, dev)
    if dST is not None:
        _check_tensor("dST", dST, (B, H, dk, dv), torch.float32, dev)
    f32 = dict(dtype=torch.float32, device=dev)
    out = {"dq": torch.empty((B, T, H, dk), **f32), "dk": torch.empty((B, T, H, dk), **f32),
           "dv": torch.empty((B, T, H, dv), **f32), "dbeta": torch.empty((B, T, H), **f32),
           "dS0": torch.empty((B, H, dk, dv), **f32),
           "dg": None if gate_layout == "none" else
           torch.empty((B, T, H, dk) if gate_layout == "channel" else (B, T, H), **f32)}
    L = _lib.lib()
    gl = _gate(gate_layout)
    if pre:
        nbytes = int(L.kda_chunk_bwd_pre_workspace_bytes(B, T, H, dk, dv, _code(q.dtype), chunk_size, gl, pre))
    else:
        nbytes = int(L.kda_chunk_bwd_workspace_bytes(B, T, H, dk, dv, _code(q.dtype), chunk_size))
    if nbytes == 0 and B * T * H > 0:
        raise _lib.KdaError(3, "kda_chunk_bwd_workspace_bytes")
    if workspace is None:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)
    args = (_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(initial_state), _ptr(dO), _ptr(dST),
            _ptr(out["dq"]), _ptr(out["dk"]), _ptr(out["dv"]), _ptr(out["dg"]), _ptr(out["dbeta"]),
            _ptr(out["dS0"]), B, T, H, dk, dv, _code(q.dtype), _ptr(workspace), workspace.numel(),
            _stream(stream, dev), chunk_size, gl)
    if pre:
        _lib.check(L.kda_chunk_bwd_pre(*args, pre), "kda_chunk_bwd_pre")
    else:
        _lib.check(L.kda_chunk_bwd(*args), "kda_chunk_bwd")
    return out


def chunk_bwd_varlen(q, k, v, g, beta, dO, cu_seqlens, initial_state=None, dST=None, chunk_size=64,
                     gate_layout="channel", workspace=None, stream=None):
    """Backward pass of chunk_fwd_varlen (kda_chunk_bwd_varlen).  q,k [T,H,dk],
    v [T,H,dv], beta [T,H], dO [T,H,dv] fp32, cu_seqlens int32 [N+1];
    initial_state and dST [N,H,dk,dv] fp32 or None.  Returns a dict of fp32
    tensors dq, dk, dv, dg (None without gates), dbeta, dS0 [N,H,dk,dv]."""
    _gate(gate_layout)
    T, H, dk = q.shape
    dv = v.shape[-1]
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("inputs must be on a GPU")
    N = cu_seqlens.numel() - 1
    if N < 0:
        raise ValueError("cu_seqlens needs at least one entry")
    _check_tensor("cu_seqlens", cu_seqlens, (N + 1,), torch.int32, dev)
    _check_tensor("k", k, (T, H, dk), q.dtype, dev)
    _check_tensor("v", v, (T, H, dv), q.dtype, dev)
    _check_gate(g, gate_layout, (T, H), dk, dev)
    _check_tensor("beta", beta, (T, H), torch.float32, dev)
    _check_tensor("dO", dO, (T, H, dv), torch.float32, dev)
    if initial_state is not None:
        _check_tensor("initial_state", initial_state, (N, H, dk, dv), torch.float32, dev)
    if dST is not None:
        _check_tensor("dST", dST, (N, H, dk, dv), torch.float32, dev)
    f32 = dict(dtype=torch.float32, device=dev)
    out = {"dq": torch.empty((T, H, dk), **f32), "dk": torch.empty((T, H, dk), **f32),
           "dv": torch.empty((T, H, dv), **f32), "dbeta": torch.empty((T, H), **f32),
           "dS0": torch.empty((N, H, dk, dv), **f32),
           "dg": None if gate_layout == "none" else
           torch.empty((T, H, dk) if gate_layout == "channel" else (T, H), **f32)}
    L = _lib.lib()
    nbytes = int(L.kda_chunk_bwd_varlen_workspace_bytes(N, T, H, dk, dv, _code(q.dtype), chunk_size))
    if nbytes == 0 and N * T * H > 0:
        raise _lib.KdaError(3, "kda_chunk_bwd_varlen_workspace_bytes")
    if workspace is None:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)
    st = L.kda_chunk_bwd_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(initial_state), _ptr(dO),
                                _ptr(dST), _ptr(out["dq"]), _ptr(out["dk"]), _ptr(out["dv"]), _ptr(out["dg"]),
                                _ptr(out["dbeta"]), _ptr(out["dS0"]), _ptr(cu_seqlens), N, T, H, dk, dv,
                                _code(q.dtype), _ptr(workspace), workspace.numel(), _stream(stream, dev), chunk_size,
                                _gate(gate_layout))
    _lib.check(st, "kda_chunk_bwd_varlen")
    return out


class ChunkPlan:
    """Pre-allocated outputs and workspace for repeated kda_chunk_fwd calls on the
    same sizes; ``run`` calls both stages, ``intra``/``chain`` one each."""

    def __init__(self, q, k, v, g, beta, initial_state=None, chunk_size=64, out_dtype=None,
                 gate_layout="channel", qk_l2norm=False, gate_act=None):
        self.args = (q, k, v, g, beta, initial_state)
        self.chunk_size = chunk_size
        self.gate_layout = gate_layout
        self.pre = _pre_flags(qk_l2norm, gate_act, g, gate_layout)
        (self.B, self.T, self.H, self.dk, self.dv, self.out_dtype, self.o, self.final_state,
         self.workspace) = _prep_chunk(q, k, v, g, beta, initial_state, chunk_size, out_dtype, None, None,
                                       gate_layout, allow_bf16_gate=True)
        # segments the chain stage runs each sequence in (1: the plain sequential chain)
        self.segments = int(_lib.lib().kda_chunk_fwd_segments(self.B, self.T, self.H, self.dk, self.dv,
                                                              _code(q.dtype), chunk_size))
        self.segmented = self.segments > 1
        # the chunk size the kernels run (C = 128 may run as 64-token chunks)
        self.chunk_used = int(_lib.lib().kda_chunk_size_used(self.dk, self.dv, _code(q.dtype), chunk_size, 0))

    def _go(self, name, stream=None):
        q, k, v, g, beta, s0 = self.args
        _call_chunk(name, q, k, v, g, beta, s0, self.o, self.final_state, self.B, self.T, self.H,
                    self.dk, self.dv, self.out_dtype, self.workspace, self.chunk_size, stream,
                    self.gate_layout, self.pre)

    def run(self, stream=None):
        self._go("kda_chunk_fwd", stream)
        return self.o, self.final_state

    def intra(self, stream=None):
        self._go("kda_chunk_intra", stream)

    def chain(self, stream=None):
        self._go("kda_chunk_chain", stream)


def decode_step(q, k, v, g, beta, state, out_dtype=None, o=None, stream=None, gate_layout="channel"):
    """One decode step (kda_decode_step / kda_decode_step_ex).  q,k [N,H,dk],
    v [N,H,dv]; g fp32 [N,H,dk] ("channel"), [N,H] ("head") or None ("none");
    beta [N,H] fp32; state [N,H,dk,dv] fp32 is updated in place.  Returns o."""
    N, H, dk = q.shape
    dv = v.shape[-1]
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("inputs must be on a GPU")
    _check_tensor("k", k, (N, H, dk), q.dtype, dev)
    _check_tensor("v", v, (N, H, dv), q.dtype, dev)
    _check_gate(g, gate_layout, (N, H), dk, dev)
    _check_tensor("beta", beta, (N, H), torch.float32, dev)
    _check_tensor("state", state, (N, H, dk, dv), torch.float32, dev)
    out_dtype = q.dtype if out_dtype is None else out_dtype
    if o is None:
        o = torch.empty((N, H, dv), dtype=out_dtype, device=dev)
    st = _lib.lib().kda_decode_step_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(state),
                                       _ptr(o), N, H, dk, dv, _code(q.dtype), _code(out_dtype),
                                       _stream(stream, dev), _gate(gate_layout))
    _lib.check(st, "kda_decode_step_ex")
    return o


def decode_tokens(q, k, v, g, beta, state, out_dtype=None, o=None, stream=None, gate_layout="channel",
                  qk_l2norm=False, gate_act=None):
    """T tokens per sequence in one call (kda_decode_tokens / _pre).  q,k
    [N,T,H,dk], v [N,T,H,dv]; g fp32 [N,T,H,dk] ("channel"), [N,T,H] ("head") or
    None ("none"); beta [N,T,H] fp32; state [N,H,dk,dv] fp32 is updated in place.
    Returns o [N,T,H,dv].  ``qk_l2norm`` and ``gate_act`` as in chunk_fwd."""
    pre = _pre_flags(qk_l2norm, gate_act, g, gate_layout)
    N, T, H, dk = q.shape
    dv = v.shape[-1]
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("inputs must be on a GPU")
    _check_tensor("k", k, (N, T, H, dk), q.dtype, dev)
    _check_tensor("v", v, (N, T, H, dv), q.dtype, dev)
    _check_gate(g, gate_layout, (N, T, H), dk, dev, allow_bf16=True)
    _check_tensor("beta", beta, (N, T, H), torch.float32, dev)
    _check_tensor("state", state, (N, H, dk, dv), torch.float32, dev)
    out_dtype = q.dtype if out_dtype is None else out_dtype
    if o is None:
        o = torch.empty((N, T, H, dv), dtype=out_dtype, device=dev)
    args = [_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(state), _ptr(o), N, T, H, dk, dv,
            _code(q.dtype), _code(out_dtype), _stream(stream, dev), _gate(gate_layout)]
    name = "kda_decode_tokens_pre" if pre else "kda_decode_tokens"
    st = getattr(_lib.lib(), name)(*(args + [pre] if pre else args))
    _lib.check(st, name)
    return o
