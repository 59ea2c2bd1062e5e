"""The oracle against what the pages and the mathematics fix (CPU only)."""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from tests import pins


def c_impl(q, k, v, g, beta, S0=None, delta=True):
    return oracle.recurrent(q, k, v, g, beta, S0, delta=delta)


def np_impl(q, k, v, g, beta, S0=None, delta=True):
    return oracle.recurrent_np(q, k, v, g, beta, S0, delta=delta)


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda p: p.__name__)
def test_pin_c_oracle(pin):
    pin(c_impl)


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda p: p.__name__)
def test_pin_numpy_twin(pin):
    pin(np_impl)


def test_twin_agrees_with_c():
    q, k, v, g, beta = pins._rand(7, 2, 50, 3, 9, 7)
    S0 = np.random.default_rng(8).standard_normal((2, 3, 9, 7))
    o1, s1 = c_impl(q, k, v, g, beta, S0)
    o2, s2 = np_impl(q, k, v, g, beta, S0)
    np.testing.assert_allclose(o1, o2, atol=1e-13)
    np.testing.assert_allclose(s1, s2, atol=1e-13)


@pytest.mark.parametrize("C", [1, 2, 16, 37, 64, 128, 256])
def test_chunked_form_equals_recurrence(C):
    """Chunk paragraph of the KimiK3 essay / explainer section 十六: any chunk size
    gives the recurrence's result; C=1 is the recurrence itself, C=T one chunk of
    masked attention.  37 leaves a partial last chunk."""
    q, k, v, g, beta = pins._rand(131, 1, 256, 2, 16, 8)
    S0 = 0.1 * np.random.default_rng(132).standard_normal((1, 2, 16, 8))
    o, S = c_impl(q, k, v, g, beta, S0)
    oc, Sc = oracle.chunked_np(q, k, v, g, beta, S0, C=C)
    np.testing.assert_allclose(oc, o, atol=1e-12)
    np.testing.assert_allclose(Sc, S, atol=1e-12)


def test_chunk_partition_example():
    """Explainer section 十六: 1024 tokens in chunks 1-64, 65-128, 129-192, ..."""
    f = json.load(open(os.path.join(pins.GOLDEN, "chunk_partition.json")))
    T, C = f["T"], f["C"]
    starts = list(range(0, T, C))
    assert len(starts) == f["n_chunks"]
    assert [[s + 1, s + C] for s in starts[:3]] == f["first_chunks_1based"]
    q, k, v, g, beta = pins._rand(141, 1, T, 1, 8, 4)
    o, S = c_impl(q, k, v, g, beta)
    oc, Sc = oracle.chunked_np(q, k, v, g, beta, C=C)
    np.testing.assert_allclose(oc, o, atol=1e-12)
    np.testing.assert_allclose(Sc, S, atol=1e-12)


def test_exact_rational():
    """fp64 oracle vs exact rational arithmetic of the same definition (alpha
    rational, g = log alpha): only rounding may differ."""
    r = np.random.default_rng(151)
    T, dk, dv = 5, 3, 3
    den = 8
    q = r.integers(-den, den + 1, (T, dk)) / den
    k = r.integers(-den, den + 1, (T, dk)) / den
    v = r.integers(-den, den + 1, (T, dv)) / den
    alpha = r.integers(1, den + 1, (T, dk)) / den
    beta = r.integers(0, den + 1, T) / den
    S0 = r.integers(-den, den + 1, (dk, dv)) / den
    to_f = lambda a: [[Fraction(x).limit_denominator(1 << 20) for x in row] for row in a]
    oe, Se = oracle.recurrent_exact(to_f(q), to_f(k), to_f(v), to_f(alpha),
                                    [Fraction(x).limit_denominator(1 << 20) for x in beta], to_f(S0))
    o, S = c_impl(q[None, :, None], k[None, :, None], v[None, :, None],
                  np.log(alpha)[None, :, None], beta[None, :, None], S0[None, None])
    np.testing.assert_allclose(o[0, :, 0], np.array(oe, dtype=float), atol=2e-14)
    np.testing.assert_allclose(S[0, 0], np.array(Se, dtype=float), atol=2e-14)


def test_u_dump_is_the_write():
    """u_t returned by the oracle is the correction written along k_t."""
    q, k, v, g, beta = pins._rand(161, 1, 6, 1, 4, 3)
    o, S, u = oracle.recurrent(q, k, v, g, beta, dump_u=True)
    _, S5 = c_impl(q[:, :5], k[:, :5], v[:, :5], g[:, :5], beta[:, :5])
    S6 = np.exp(g[0, 5, 0])[:, None] * S5[0, 0] + np.outer(k[0, 5, 0], u[0, 5, 0])
    np.testing.assert_allclose(S[0, 0], S6, atol=1e-14)


def test_threads_reported():
    q, k, v, g, beta = pins._rand(171, 1, 4, 4, 4, 4)
    oracle.recurrent(q, k, v, g, beta, nthreads=2)
    assert oracle.last_threads() == 2
