"""Each plausible mistake in the recurrence fails at least one oracle pin.

The mistakes are planted in CPU-only copies of the definition below (never in
the GPU path): a dropped decay, the decay after the read or after the write, the
gate applied to value columns, the output read before the write, a sign error in
the correction, the read without the transpose, beta dropped or applied to the
value only, and the gate exponent's sign flipped.
"""
import numpy as np
import pytest

from tests import pins


def make_mutant(kind):
    def impl(q, k, v, g, beta, S0=None, delta=True):
        B, T, H, dk = q.shape
        dv = v.shape[-1]
        S = np.zeros((B, H, dk, dv)) if S0 is None else np.array(S0, dtype=float)
        o = np.empty((B, T, H, dv))
        for t in range(T):
            a = np.exp(g[:, t])
            if kind == "gate_sign":
                a = np.exp(-g[:, t])
            decay = (lambda M: a[..., None] * M)
            if kind == "gate_on_columns":
                decay = (lambda M: M * a[..., None, :] if dk == dv else M * a.mean(-1)[..., None, None])
            if kind not in ("no_decay", "decay_after_read", "decay_after_write"):
                S = decay(S)
            if kind == "transposed_read" and dk == dv:
                r = np.einsum("bhj,bhcj->bhc", k[:, t], S)
            else:
                r = np.einsum("bhc,bhcj->bhj", k[:, t], S)
            if not delta:
                r = 0.0
            if kind == "decay_after_read":
                S = decay(S)
            bt = beta[:, t, :, None]
            if kind == "no_beta":
                u = v[:, t] - r
            elif kind == "beta_on_value_only":
                u = bt * v[:, t] - r
            elif kind == "error_sign":
                u = bt * (r - v[:, t])
            else:
                u = bt * (v[:, t] - r)
            o_pre = np.einsum("bhc,bhcj->bhj", q[:, t], S)
            S = S + k[:, t, :, :, None] * u[:, :, None, :]
            if kind == "decay_after_write":
                S = decay(S)
            o[:, t] = o_pre if kind == "output_before_write" else np.einsum("bhc,bhcj->bhj", q[:, t], S)
        return o, S
    return impl


KINDS = ["no_decay", "decay_after_read", "decay_after_write", "gate_on_columns",
         "output_before_write", "error_sign", "transposed_read", "no_beta",
         "beta_on_value_only", "gate_sign"]


def test_unmutated_copy_passes_all_pins():
    impl = make_mutant("none")
    for pin in pins.ALL_PINS:
        pin(impl)


@pytest.mark.parametrize("kind", KINDS)
def test_mutant_is_caught(kind):
    impl = make_mutant(kind)
    failed = []
    with np.errstate(all="ignore"):
        for pin in pins.ALL_PINS:
            try:
                pin(impl)
            except (AssertionError, FloatingPointError, ValueError):
                failed.append(pin.__name__)
    assert failed, f"mutant {kind} passed every pin"
