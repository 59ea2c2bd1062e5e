"""Shared helpers for GPU-vs-oracle parity checks.

Tolerance (per output tensor X): max |X_gpu - X_ref| <= tol * max(1, max |X_ref|),
tol = 1e-4 when q,k,v are fp32 and 2e-2 when they are bf16 (state fp32)."""
import numpy as np
import torch

TOL = {torch.float32: 1e-4, torch.bfloat16: 2e-2}


def to64(x):
    if isinstance(x, torch.Tensor):
        return x.detach().to("cpu", torch.float64).numpy()
    return np.asarray(x, dtype=np.float64)


def max_err(x, ref):
    x, ref = to64(x), to64(ref)
    assert x.shape == ref.shape, (x.shape, ref.shape)
    return float(np.max(np.abs(x - ref))) if x.size else 0.0


def assert_close(name, x, ref, tol):
    x64, r64 = to64(x), to64(ref)
    err = max_err(x64, r64)
    scale = max(1.0, float(np.max(np.abs(r64))) if r64.size else 1.0)
    assert np.all(np.isfinite(x64)), f"{name}: non-finite values"
    assert err <= tol * scale, f"{name}: max abs err {err:.3e} > {tol:.1e} * {scale:.3g}"
    return err


def cuda(d):
    """Move a dict of CPU tensors (None allowed) to cuda:0."""
    return {k: (None if v is None else v.to("cuda:0").contiguous()) for k, v in d.items()}
