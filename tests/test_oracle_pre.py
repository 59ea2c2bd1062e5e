"""Pins of the oracle's pre-processing functions (CPU): the L2 normalisation of
q and k rows and the log-gate -softplus(a) of the method's workloads, and their
vector-Jacobian products (pinned by central differences of the functions
themselves, invariants and worked examples)."""
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


def _central_difference(f, x, dy, eps):
    """d/dt sum(dy * f(x + t E)) at t = 0 for every basis direction E: the
    gradient by central differences, one coordinate at a time."""
    grad = np.zeros_like(x)
    it = np.nditer(x, flags=["multi_index"])
    for _ in it:
        i = it.multi_index
        xp, xm = x.copy(), x.copy()
        xp[i] += eps
        xm[i] -= eps
        grad[i] = np.sum(dy * (f(xp) - f(xm))) / (2 * eps)
    return grad


def test_l2_normalize_vjp_finite_differences_and_invariants():
    rs = np.random.default_rng(3)
    x = rs.standard_normal((3, 2, 8)) * rs.uniform(0.1, 10.0, (3, 2, 1))
    dy = rs.standard_normal(x.shape)
    dx = oracle.l2_normalize_vjp(x, dy)
    fd = _central_difference(oracle.l2_normalize, x, dy, 1e-6)
    assert np.allclose(dx, fd, rtol=0, atol=1e-7 * np.abs(fd).max())
    # the normalisation does not change along x: the gradient is orthogonal to x
    assert np.allclose(np.sum(dx * x, axis=-1), 0.0, rtol=0, atol=1e-13 * np.abs(x).max() * np.abs(dx).max())
    # scaling x by c scales the gradient by 1/c
    assert np.allclose(oracle.l2_normalize_vjp(4.0 * x, dy), dx / 4.0, rtol=1e-13, atol=0)
    # a cotangent along y = x/|x| has no effect
    y = oracle.l2_normalize(x)
    assert np.allclose(oracle.l2_normalize_vjp(x, 2.5 * y), 0.0, rtol=0, atol=1e-15)
    # worked example: x = (3, 4), dy = (1, 0): (I - y y^T)/5 e1 = (1 - 0.36, -0.48)/5
    assert np.allclose(oracle.l2_normalize_vjp(np.array([3.0, 4.0]), np.array([1.0, 0.0])),
                       [0.64 / 5, -0.48 / 5], rtol=0, atol=1e-16)
    # a zero row gets zero
    assert np.array_equal(oracle.l2_normalize_vjp(np.zeros((1, 4)), np.ones((1, 4))), np.zeros((1, 4)))


def test_gate_softplus_vjp_finite_differences_and_closed_forms():
    rs = np.random.default_rng(4)
    a = rs.standard_normal((4, 5)) * 4
    dg = rs.standard_normal(a.shape)
    da = oracle.gate_softplus_vjp(a, dg)
    fd = _central_difference(oracle.gate_softplus, a, dg, 1e-6)
    assert np.allclose(da, fd, rtol=0, atol=1e-8)
    # at a = 0 the slope is -1/2; far right -1; far left ~ -e^a
    v = oracle.gate_softplus_vjp(np.array([0.0, 60.0, -60.0, 800.0, -800.0]), np.ones(5))
    assert v[0] == -0.5 and v[1] == -1.0
    assert abs(v[2] + np.exp(-60.0)) < 1e-40
    assert v[3] == -1.0 and v[4] == 0.0 or abs(v[4]) < 1e-300
    # sigmoid(a) + sigmoid(-a) = 1, so the slopes at a and at -a sum to -1
    b = rs.standard_normal(1000) * 8
    one = np.ones_like(b)
    assert np.allclose(oracle.gate_softplus_vjp(b, one) + oracle.gate_softplus_vjp(-b, one), -1.0,
                       rtol=0, atol=1e-15)
