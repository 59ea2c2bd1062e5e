"""Pins of the oracle's backward (the adjoint of the recurrence), CPU only.

(1) Central finite differences of L = sum(dO * o) + sum(dST * S_T) on tiny
inputs, every input entry; (2) an independent reverse-mode derivative: torch
autograd through a plain fp64 loop written from the definition; (3) the
checkpoint segment length does not change the result."""
import numpy as np
import pytest
import torch

import oracle


def _inputs(seed, B, T, H, dk, dv, gmu=1.0):
    rs = np.random.default_rng(seed)
    unit = lambda x: x / np.linalg.norm(x, axis=-1, keepdims=True)
    d = dict(q=unit(rs.standard_normal((B, T, H, dk))), k=unit(rs.standard_normal((B, T, H, dk))),
             v=rs.standard_normal((B, T, H, dv)), g=-np.logaddexp(0, rs.standard_normal((B, T, H, dk)) + gmu),
             beta=1 / (1 + np.exp(-rs.standard_normal((B, T, H)))), S0=0.3 * rs.standard_normal((B, H, dk, dv)))
    dO = rs.standard_normal((B, T, H, dv))
    dST = rs.standard_normal((B, H, dk, dv))
    return d, dO, dST


def _loss(d, dO, dST):
    o, S = oracle.recurrent(d["q"], d["k"], d["v"], d["g"], d["beta"], d["S0"])
    return float(np.sum(o * dO) + np.sum(S * dST))


def test_backward_finite_differences():
    d, dO, dST = _inputs(1, 1, 5, 2, 3, 2)
    grads = oracle.backward(d["q"], d["k"], d["v"], d["g"], d["beta"], d["S0"], dO, dST, seg=2)
    names = {"q": "dq", "k": "dk", "v": "dv", "g": "dg", "beta": "dbeta", "S0": "dS0"}
    eps = 1e-6
    for x, gname in names.items():
        num = np.zeros_like(d[x])
        for idx in np.ndindex(d[x].shape):
            dp = {key: val.copy() for key, val in d.items()}
            dm = {key: val.copy() for key, val in d.items()}
            dp[x][idx] += eps
            dm[x][idx] -= eps
            num[idx] = (_loss(dp, dO, dST) - _loss(dm, dO, dST)) / (2 * eps)
        np.testing.assert_allclose(grads[gname], num, atol=1e-7, rtol=1e-6, err_msg=gname)


def _torch_loop(q, k, v, g, beta, S0):
    B, T, H, dk = q.shape
    outs = []
    S = S0
    for t in range(T):
        a = torch.exp(g[:, t])                                   # [B,H,dk]
        Sp = a[..., None] * S
        r = torch.einsum("bhc,bhcj->bhj", k[:, t], Sp)
        u = beta[:, t, :, None] * (v[:, t] - r)
        S = Sp + k[:, t, :, :, None] * u[:, :, None, :]
        outs.append(torch.einsum("bhc,bhcj->bhj", q[:, t], S))
    return torch.stack(outs, dim=1), S


def test_backward_matches_autograd_of_a_plain_loop():
    d, dO, dST = _inputs(2, 2, 37, 3, 8, 6, gmu=0.5)
    t = {key: torch.tensor(val, dtype=torch.float64, requires_grad=True) for key, val in d.items()}
    o, S = _torch_loop(t["q"], t["k"], t["v"], t["g"], t["beta"], t["S0"])
    L = (o * torch.tensor(dO)).sum() + (S * torch.tensor(dST)).sum()
    auto = torch.autograd.grad(L, [t[key] for key in ("q", "k", "v", "g", "beta", "S0")])
    grads = oracle.backward(d["q"], d["k"], d["v"], d["g"], d["beta"], d["S0"], dO, dST, seg=8)
    for name, ref in zip(("dq", "dk", "dv", "dg", "dbeta", "dS0"), auto):
        np.testing.assert_allclose(grads[name], ref.numpy(), atol=1e-11, rtol=1e-9, err_msg=name)


@pytest.mark.parametrize("seg", [1, 7, 64, 1000])
def test_backward_segment_length_does_not_matter(seg):
    d, dO, dST = _inputs(3, 1, 50, 2, 6, 5)
    ref = oracle.backward(d["q"], d["k"], d["v"], d["g"], d["beta"], d["S0"], dO, dST, seg=50)
    got = oracle.backward(d["q"], d["k"], d["v"], d["g"], d["beta"], d["S0"], dO, dST, seg=seg)
    for name in ref:
        np.testing.assert_allclose(got[name], ref[name], atol=1e-12, rtol=1e-12, err_msg=name)


def test_backward_without_cotangents_is_zero_and_dS0_alone():
    d, dO, dST = _inputs(4, 1, 6, 1, 4, 3)
    z = oracle.backward(d["q"], d["k"], d["v"], d["g"], d["beta"], d["S0"], None, None)
    assert all(np.all(val == 0) for val in z.values())
    # with alpha = 1 and beta = 0 the state passes through unchanged: dS0 = dST + sum_t q_t dO_t^T
    d2 = dict(d); d2["g"] = np.zeros_like(d["g"]); d2["beta"] = np.zeros_like(d["beta"])
    gr = oracle.backward(d2["q"], d2["k"], d2["v"], d2["g"], d2["beta"], d2["S0"], dO, dST)
    want = dST + np.einsum("bthc,bthj->bhcj", d2["q"], dO)
    np.testing.assert_allclose(gr["dS0"], want, atol=1e-13)
    assert np.all(gr["dv"] == 0)
