"""ctypes loader for libkda.so (the C ABI declared in include/kda.h).

The library is built in-tree by ``__graft_entry__.build()``; there is no fallback:
if it is missing every call raises."""
from __future__ import annotations

import ctypes
import os

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG_DIR, "libkda.so")

F32, BF16 = 0, 1
NOALLOC_WORKSPACE_MAX = 128 << 20                # KDA_NOALLOC_WORKSPACE_MAX in kda.h
GATE = {"channel": 0, "head": 1, "none": 2}     # kda_gate_layout_t
PRE_QK_L2NORM, PRE_GATE_SOFTPLUS, PRE_GATE_BF16 = 1, 2, 4   # kda_pre_flags_t
STATUS = {0: "KDA_OK", 1: "KDA_ERR_NULL", 2: "KDA_ERR_SHAPE", 3: "KDA_ERR_UNSUPPORTED",
          4: "KDA_ERR_MISALIGNED", 5: "KDA_ERR_WORKSPACE", 6: "KDA_ERR_ALIAS", 7: "KDA_ERR_HIP"}

# Every entry point include/kda.h declares.
SYMBOLS = ("kda_abi_version", "kda_status_string", "kda_chunk_fwd_workspace_bytes",
           "kda_chunk_fwd", "kda_chunk_intra", "kda_chunk_chain", "kda_decode_step",
           "kda_chunk_fwd_ex", "kda_chunk_intra_ex", "kda_decode_step_ex", "kda_decode_tokens",
           "kda_chunk_fwd_varlen", "kda_chunk_varlen_workspace_bytes",
           "kda_chunk_bwd", "kda_chunk_bwd_workspace_bytes",
           "kda_chunk_fwd_pre", "kda_chunk_intra_pre", "kda_decode_tokens_pre",
           "kda_chunk_bwd_varlen", "kda_chunk_bwd_varlen_workspace_bytes",
           "kda_chunk_bwd_pre", "kda_chunk_bwd_pre_workspace_bytes", "kda_chunk_fwd_segments",
           "kda_chunk_fwd_noalloc", "kda_chunk_size_used")


class KdaError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {STATUS.get(status, status)} ({status_string(status)})")


_LIB = None
_vp, _ci, _sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
_CHUNK_ARGS = [_vp] * 8 + [_ci] * 7 + [_vp, _sz, _vp, _ci]


def lib() -> ctypes.CDLL:
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build()")
        L = ctypes.CDLL(LIB_PATH)
        L.kda_abi_version.argtypes, L.kda_abi_version.restype = [], _ci
        L.kda_status_string.argtypes, L.kda_status_string.restype = [_ci], ctypes.c_char_p
        L.kda_chunk_fwd_workspace_bytes.argtypes = [_ci] * 7
        L.kda_chunk_fwd_workspace_bytes.restype = _sz
        L.kda_chunk_fwd_segments.argtypes, L.kda_chunk_fwd_segments.restype = [_ci] * 7, _ci
        L.kda_chunk_fwd_noalloc.argtypes = [_vp] * 8 + [_ci] * 7 + [_vp, _ci, _ci]
        L.kda_chunk_fwd_noalloc.restype = _ci
        L.kda_chunk_size_used.argtypes, L.kda_chunk_size_used.restype = [_ci] * 5, _ci
        for name in ("kda_chunk_fwd", "kda_chunk_intra", "kda_chunk_chain"):
            fn = getattr(L, name)
            fn.argtypes, fn.restype = _CHUNK_ARGS, _ci
        for name in ("kda_chunk_fwd_ex", "kda_chunk_intra_ex"):
            fn = getattr(L, name)
            fn.argtypes, fn.restype = _CHUNK_ARGS + [_ci], _ci
        for name in ("kda_chunk_fwd_pre", "kda_chunk_intra_pre"):
            fn = getattr(L, name)
            fn.argtypes, fn.restype = _CHUNK_ARGS + [_ci, _ci], _ci
        L.kda_decode_step.argtypes = [_vp] * 7 + [_ci] * 6 + [_vp]
        L.kda_decode_step.restype = _ci
        L.kda_decode_step_ex.argtypes = [_vp] * 7 + [_ci] * 6 + [_vp, _ci]
        L.kda_decode_step_ex.restype = _ci
        L.kda_decode_tokens.argtypes = [_vp] * 7 + [_ci] * 7 + [_vp, _ci]
        L.kda_decode_tokens.restype = _ci
        L.kda_decode_tokens_pre.argtypes = [_vp] * 7 + [_ci] * 7 + [_vp, _ci, _ci]
        L.kda_decode_tokens_pre.restype = _ci
        L.kda_chunk_fwd_varlen.argtypes = [_vp] * 9 + [_ci] * 7 + [_vp, _sz, _vp, _ci, _ci]
        L.kda_chunk_fwd_varlen.restype = _ci
        L.kda_chunk_varlen_workspace_bytes.argtypes = [_ci] * 7
        L.kda_chunk_varlen_workspace_bytes.restype = _sz
        L.kda_chunk_bwd.argtypes = [_vp] * 14 + [_ci] * 6 + [_vp, _sz, _vp, _ci, _ci]
        L.kda_chunk_bwd.restype = _ci
        L.kda_chunk_bwd_workspace_bytes.argtypes = [_ci] * 7
        L.kda_chunk_bwd_workspace_bytes.restype = _sz
        L.kda_chunk_bwd_varlen.argtypes = [_vp] * 15 + [_ci] * 6 + [_vp, _sz, _vp, _ci, _ci]
        L.kda_chunk_bwd_varlen.restype = _ci
        L.kda_chunk_bwd_varlen_workspace_bytes.argtypes = [_ci] * 7
        L.kda_chunk_bwd_varlen_workspace_bytes.restype = _sz
        L.kda_chunk_bwd_pre.argtypes = [_vp] * 14 + [_ci] * 6 + [_vp, _sz, _vp, _ci, _ci, _ci]
        L.kda_chunk_bwd_pre.restype = _ci
        L.kda_chunk_bwd_pre_workspace_bytes.argtypes = [_ci] * 9
        L.kda_chunk_bwd_pre_workspace_bytes.restype = _sz
        _LIB = L
    return _LIB


def status_string(status: int) -> str:
    try:
        return lib().kda_status_string(int(status)).decode()
    except RuntimeError:
        return "?"


def check(status: int, where: str) -> None:
    if status != 0:
        raise KdaError(status, where)
