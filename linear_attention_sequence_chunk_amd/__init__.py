"""libkda: MI355X (gfx950) kernels for the Kimi Delta Attention / gated delta-rule
state update, behind a C ABI (include/kda.h) with a thin ctypes binding."""
