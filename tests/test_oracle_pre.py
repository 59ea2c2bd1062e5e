"""Pins of the oracle's pre-processing functions (CPU): the L2 normalisation of
q and k rows and the log-gate -softplus(a) of the method's workloads."""
import numpy as np

import oracle


def test_l2_normalize_worked_example_and_invariants():
    x = np.array([[3.0, 4.0], [0.0, 0.0], [-1.0, 0.0]])
    y = oracle.l2_normalize(x)
    assert np.array_equal(y[0], [0.6, 0.8])           # the 3-4-5 triangle
    assert np.array_equal(y[1], [0.0, 0.0])           # a zero row stays zero
    assert np.array_equal(y[2], [-1.0, 0.0])
    rs = np.random.default_rng(1)
    z = rs.standard_normal((5, 7, 64)) * rs.uniform(0.01, 100.0, (5, 7, 1))
    u = oracle.l2_normalize(z)
    assert np.allclose(np.linalg.norm(u, axis=-1), 1.0, rtol=0, atol=1e-14)
    assert np.allclose(u * np.linalg.norm(z, axis=-1, keepdims=True), z, rtol=1e-14, atol=0)
    assert np.allclose(oracle.l2_normalize(3.5 * z), u, rtol=0, atol=1e-15)      # scale invariant
    assert np.array_equal(oracle.l2_normalize(-z), -u)                           # odd


def test_gate_softplus_closed_forms():
    g = oracle.gate_softplus(np.array([0.0, 50.0, -50.0, 800.0, -800.0]))
    assert g[0] == -np.log(2.0)
    assert abs(g[1] + 50.0) < 1e-13                   # -softplus(a) -> -a for large a
    assert abs(g[2] + np.exp(-50.0)) < 1e-30          # -> -e^a for very negative a
    assert g[3] == -800.0 and g[4] == -0.0 or abs(g[4]) < 1e-300   # no overflow either way
    a = np.random.default_rng(2).standard_normal(1000) * 6
    # softplus(a) - softplus(-a) = a
    assert np.allclose(oracle.gate_softplus(-a) - oracle.gate_softplus(a), a, rtol=0, atol=1e-13)
    # alpha = e^g is the logistic function of -a
    assert np.allclose(np.exp(oracle.gate_softplus(a)), 1.0 / (1.0 + np.exp(a)), rtol=1e-14, atol=0)
    assert np.all(np.diff(oracle.gate_softplus(np.sort(a))) <= 0)                # decreasing
