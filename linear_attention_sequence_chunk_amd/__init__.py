"""libkda: MI355X (gfx950) kernels for the Kimi Delta Attention / gated delta-rule
state update, behind a C ABI (include/kda.h) with a thin ctypes binding.

    from linear_attention_sequence_chunk_amd import chunk_fwd, decode_step
"""
from .api import (ChunkPlan, chunk_bwd, chunk_bwd_varlen, chunk_fwd, chunk_fwd_noalloc, chunk_fwd_varlen, decode_step,  # noqa: F401
                  decode_tokens, workspace_bytes)
from ._lib import KdaError  # noqa: F401
