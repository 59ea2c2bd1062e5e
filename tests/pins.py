"""Pins for the oracle: checks against what the pages and the mathematics fix.

Each pin takes an implementation ``impl(q, k, v, g, beta, S0=None, delta=True)
-> (o, S_T)`` working on fp64 numpy arrays ([B,T,H,d] layout) and raises
AssertionError when it disagrees.  tests/test_oracle_pins.py runs every pin on
the oracle; tests/test_pin_power.py runs them on deliberately broken variants
of the recurrence to show that each plausible mistake fails at least one pin.
"""
from __future__ import annotations

import json
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _unit(x):
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def _rand(seed, B, T, H, dk, dv, gate_mu=2.0):
    r = np.random.default_rng(seed)
    q = _unit(r.standard_normal((B, T, H, dk)))
    k = _unit(r.standard_normal((B, T, H, dk)))
    v = r.standard_normal((B, T, H, dv))
    beta = 1.0 / (1.0 + np.exp(-r.standard_normal((B, T, H))))
    g = -np.logaddexp(0.0, r.standard_normal((B, T, H, dk)) + gate_mu)
    return q, k, v, g, beta


def _seq(tokens, dk, dv):
    """Pack a list of per-token dicts (q, k, v, g, beta) into [1,T,1,d] arrays."""
    T = len(tokens)
    q = np.zeros((1, T, 1, dk)); k = np.zeros((1, T, 1, dk)); v = np.zeros((1, T, 1, dv))
    g = np.zeros((1, T, 1, dk)); beta = np.zeros((1, T, 1))
    for t, tok in enumerate(tokens):
        q[0, t, 0] = tok.get("q", 0.0); k[0, t, 0] = tok.get("k", 0.0)
        v[0, t, 0] = tok.get("v", 0.0); g[0, t, 0] = tok.get("g", 0.0)
        beta[0, t, 0] = tok.get("beta", 0.0)
    return q, k, v, g, beta


# ----------------------------------------------------------------------------- pins
def pin_overwrite_narrative(impl):
    """Golden: explainer sections 一/五/六, four status updates to one key."""
    f = _golden("overwrite_narrative.json")
    key = np.array(f["key"])
    toks = [dict(k=key, v=np.array(val), beta=1.0) for val in f["values"]]
    toks.append(dict(q=key, beta=0.0))
    q, k, v, g, beta = _seq(toks, f["dk"], f["dv"])
    o, _ = impl(q, k, v, g, beta, None, True)
    np.testing.assert_allclose(o[0, -1, 0], f["expected_delta"], atol=1e-14)
    o, _ = impl(q, k, v, g, beta, None, False)
    np.testing.assert_allclose(o[0, -1, 0], f["expected_additive"], atol=1e-14)


def pin_key_collision(impl):
    """Golden + closed form: explainer section 十一 (similar keys overwrite).
    Write (k_A, v_A, beta_A) then (k_B, v_B, beta_B), read with k_A:
    beta_A (1 - beta_B c^2) v_A + beta_B c v_B."""
    f = _golden("key_collision.json")
    dk, dv = f["dk"], f["dv"]
    vA, vB = np.eye(dv)[0], np.eye(dv)[1]
    cases = [(c["cos"], 1.0, 1.0, np.array(c["expected"])) for c in f["cases"]]
    for c in (0.3, 0.8, -0.6):
        for bA, bB in ((1.0, 1.0), (0.5, 0.9), (0.9, 0.25)):
            cases.append((c, bA, bB, bA * (1 - bB * c * c) * vA + bB * c * vB))
    for c, bA, bB, expect in cases:
        kA = np.eye(dk)[0]
        kB = c * np.eye(dk)[0] + np.sqrt(max(0.0, 1 - c * c)) * np.eye(dk)[1]
        toks = [dict(k=kA, v=vA, beta=bA), dict(k=kB, v=vB, beta=bB), dict(q=kA, beta=0.0)]
        q, k, v, g, beta = _seq(toks, dk, dv)
        o, _ = impl(q, k, v, g, beta, None, True)
        np.testing.assert_allclose(o[0, -1, 0], expect, atol=1e-14)


def pin_alpha_zero_clears(impl):
    """Gated DeltaNet paragraph of the KimiK3 essay: alpha = 0 clears memory.
    With g = -inf on every channel at token t0: o_t0 = beta (q.k) v, and the
    outputs from t0 on do not depend on anything before t0 (bitwise)."""
    B, T, H, dk, dv, t0 = 1, 24, 2, 8, 6, 9
    q, k, v, g, beta = _rand(11, B, T, H, dk, dv)
    g[:, t0] = -np.inf
    S0 = np.random.default_rng(12).standard_normal((B, H, dk, dv))
    o, S = impl(q, k, v, g, beta, S0, True)
    expect = beta[:, t0, :, None] * np.einsum("bhc,bhc->bh", q[:, t0], k[:, t0])[..., None] * v[:, t0]
    np.testing.assert_allclose(o[:, t0], expect, atol=1e-14)
    r = np.random.default_rng(13)
    q2, k2, v2, g2, b2 = (x.copy() for x in (q, k, v, g, beta))
    for x in (q2, k2, v2):
        x[:, :t0] = r.standard_normal(x[:, :t0].shape)
    g2[:, :t0] = -r.random(g2[:, :t0].shape)
    b2[:, :t0] = r.random(b2[:, :t0].shape)
    o2, S2 = impl(q2, k2, v2, g2, b2, 2.0 * S0, True)
    assert np.array_equal(o2[:, t0:], o[:, t0:]) and np.array_equal(S2, S)


def pin_alpha_zero_per_channel(impl):
    """Kimi Linear paragraph: the gate acts per key channel.  One token whose
    gate is -inf on a subset of channels: the rows of S0 in those channels have
    no influence at all (bitwise), while the other rows do."""
    B, T, H, dk, dv = 1, 1, 1, 6, 6
    q, k, v, g, beta = _rand(21, B, T, H, dk, dv)
    cleared = np.array([1, 4])
    g[0, 0, 0, cleared] = -np.inf
    S0 = np.random.default_rng(22).standard_normal((B, H, dk, dv))
    o, S = impl(q, k, v, g, beta, S0, True)
    S1 = S0.copy(); S1[0, 0, cleared, :] += 5.0
    o1, Sb = impl(q, k, v, g, beta, S1, True)
    assert np.array_equal(o1, o) and np.array_equal(Sb, S)
    S2 = S0.copy(); S2[0, 0, 0, :] += 5.0            # a channel that is not cleared
    o2, _ = impl(q, k, v, g, beta, S2, True)
    assert not np.allclose(o2, o)


def pin_beta_zero(impl):
    """beta = 0 (learning rate 0 in the explainer's section 六 update): the state
    only decays, row c by exp(sum of g_c): S_t = Diag(exp(G_t)) S0,
    o_t = S_t^T q_t; v has no influence (bitwise).  dk != dv and dk == dv."""
    for dk, dv in ((5, 3), (6, 6)):
        B, T, H = 2, 12, 2
        q, k, v, g, beta = _rand(31 + dk, B, T, H, dk, dv, gate_mu=0.0)
        beta[:] = 0.0
        S0 = np.random.default_rng(32).standard_normal((B, H, dk, dv))
        o, S = impl(q, k, v, g, beta, S0, True)
        G = np.cumsum(g, axis=1)                                  # [B,T,H,dk]
        St = np.exp(G)[..., None] * S0[:, None]                   # [B,T,H,dk,dv]
        np.testing.assert_allclose(S, St[:, -1], rtol=1e-13, atol=1e-15)
        np.testing.assert_allclose(o, np.einsum("bthc,bthcj->bthj", q, St), rtol=1e-12, atol=1e-14)
        o2, S2 = impl(q, k, 3.0 * v + 1.0, g, beta, S0, True)
        assert np.array_equal(o2, o) and np.array_equal(S2, S)


def pin_additive_closed_form(impl):
    """Section 五 of the explainer (Memory = Memory + Key x Value) with the gate
    and beta: dropping the read gives
    o_t = sum_c q_tc e^{G_tc} S0[c,:] + sum_{i<=t} beta_i (sum_c q_tc k_ic e^{G_tc - G_ic}) v_i,
    G the cumulative log-gate from the sequence start.  With g = 0, beta = 1,
    S0 = 0 it is causal linear attention, tril(Q K^T) V."""
    B, T, H, dk, dv = 1, 20, 2, 5, 4
    q, k, v, g, beta = _rand(41, B, T, H, dk, dv, gate_mu=0.0)
    S0 = np.random.default_rng(42).standard_normal((B, H, dk, dv))
    o, _ = impl(q, k, v, g, beta, S0, False)
    G = np.cumsum(g, axis=1)
    expect = np.zeros_like(o)
    for b in range(B):
        for h in range(H):
            for t in range(T):
                acc = (q[b, t, h] * np.exp(G[b, t, h])) @ S0[b, h]
                for i in range(t + 1):
                    w = np.sum(q[b, t, h] * k[b, i, h] * np.exp(G[b, t, h] - G[b, i, h]))
                    acc = acc + beta[b, i, h] * w * v[b, i, h]
                expect[b, t, h] = acc
    np.testing.assert_allclose(o, expect, rtol=1e-12, atol=1e-13)
    g0 = np.zeros_like(g); b1 = np.ones_like(beta)
    o, _ = impl(q, k, v, g0, b1, None, False)
    for h in range(H):
        la = np.tril(q[0, :, h] @ k[0, :, h].T) @ v[0, :, h]
        np.testing.assert_allclose(o[0, :, h], la, rtol=1e-12, atol=1e-13)


def pin_unit_key_self_recall(impl):
    """Write then read with the same unit key at beta = 1: the output is exactly
    the value just written (q_t = k_t => o_t = v_t), whatever the gates and the
    history.  Fixes the decay -> read -> error -> write order of section 八 and
    the post-write output."""
    B, T, H, dk, dv = 2, 30, 2, 7, 5
    q, k, v, g, beta = _rand(51, B, T, H, dk, dv)
    beta[:] = 1.0
    q = k.copy()
    S0 = np.random.default_rng(52).standard_normal((B, H, dk, dv))
    o, _ = impl(q, k, v, g, beta, S0, True)
    np.testing.assert_allclose(o, v, atol=1e-12)


def pin_orthonormal_recall(impl):
    """Delta rule with alpha = 1, beta = 1 and m <= dk orthonormal keys written
    once each: querying key j returns v_j exactly (probe tokens, beta = 0)."""
    dk, dv, m = 8, 5, 6
    r = np.random.default_rng(61)
    Kq, _ = np.linalg.qr(r.standard_normal((dk, dk)))
    keys = Kq[:, :m].T
    vals = r.standard_normal((m, dv))
    toks = [dict(k=keys[j], v=vals[j], beta=1.0) for j in range(m)]
    toks += [dict(q=keys[j], beta=0.0) for j in range(m)]
    q, k, v, g, beta = _seq(toks, dk, dv)
    o, _ = impl(q, k, v, g, beta, None, True)
    np.testing.assert_allclose(o[0, m:, 0], vals, atol=1e-13)


def pin_kaczmarz_least_norm(impl):
    """With alpha = 1 and unit keys, the delta rule is a projection (Kaczmarz)
    step for the equations S^T k_i = v_i; from S0 = 0 and cycling over m < dk
    independent keys it converges to the minimum-norm solution, which numpy's
    least-squares routine gives directly.  beta in (0, 2) is the relaxed step."""
    dk, dv, m, sweeps = 12, 4, 5, 150
    r = np.random.default_rng(71)
    keys = _unit(r.standard_normal((m, dk)))
    vals = r.standard_normal((m, dv))
    ref = np.linalg.lstsq(keys, vals, rcond=None)[0]               # [dk, dv]
    for bt in (1.0, 0.7, 1.4):
        toks = [dict(k=keys[i], v=vals[i], beta=bt) for _ in range(sweeps) for i in range(m)]
        q, k, v, g, beta = _seq(toks, dk, dv)
        _, S = impl(q, k, v, g, beta, None, True)
        np.testing.assert_allclose(S[0, 0], ref, atol=1e-10)


def pin_ogd_gradient(impl):
    """Online-gradient-descent reading (cnnetsun post): the write is one step of
    gradient descent with rate beta on L(S) = 1/2 ||S^T k - v||^2 taken at the
    decayed state.  Checked against central finite differences (alpha = 1)."""
    dk, dv = 6, 4
    r = np.random.default_rng(81)
    S0 = r.standard_normal((1, 1, dk, dv))
    kk = _unit(r.standard_normal(dk)); vv = r.standard_normal(dv); bt = 0.6
    q, k, v, g, beta = _seq([dict(k=kk, v=vv, beta=bt, q=np.ones(dk))], dk, dv)
    _, S = impl(q, k, v, g, beta, S0, True)

    def loss(Sm):
        e = Sm.T @ kk - vv
        return 0.5 * float(e @ e)

    grad = np.zeros((dk, dv)); h = 1e-6
    for c in range(dk):
        for j in range(dv):
            Sp = S0[0, 0].copy(); Sp[c, j] += h
            Sm = S0[0, 0].copy(); Sm[c, j] -= h
            grad[c, j] = (loss(Sp) - loss(Sm)) / (2 * h)
    np.testing.assert_allclose(S[0, 0] - S0[0, 0], -bt * grad, atol=1e-8)


def pin_decode_identity(impl):
    """One-pass decode form: o = S^T(alpha*q) + (q.k) u, u = beta (v - S^T(alpha*k))."""
    B, H, dk, dv = 3, 2, 7, 5
    q, k, v, g, beta = _rand(91, B, 1, H, dk, dv)
    S0 = np.random.default_rng(92).standard_normal((B, H, dk, dv))
    o, S = impl(q, k, v, g, beta, S0, True)
    a = np.exp(g[:, 0])
    u = beta[:, 0, :, None] * (v[:, 0] - np.einsum("bhc,bhcj->bhj", a * k[:, 0], S0))
    expect = np.einsum("bhc,bhcj->bhj", a * q[:, 0], S0) + np.einsum("bhc,bhc->bh", q[:, 0], k[:, 0])[..., None] * u
    np.testing.assert_allclose(o[:, 0], expect, atol=1e-13)
    np.testing.assert_allclose(S, a[..., None] * S0 + k[:, 0, :, :, None] * u[:, :, None, :], atol=1e-13)


def pin_linearity_columns(impl):
    """For fixed q, k, g, beta the map (v, S0) -> (o, S_T) is linear, and value
    column j of the outputs depends only on column j of v and S0 (bitwise)."""
    B, T, H, dk, dv = 1, 16, 2, 5, 6
    q, k, v, g, beta = _rand(101, B, T, H, dk, dv)
    r = np.random.default_rng(102)
    S0 = r.standard_normal((B, H, dk, dv)); v2 = r.standard_normal(v.shape); S02 = r.standard_normal(S0.shape)
    o1, s1 = impl(q, k, v, g, beta, S0, True)
    o2, s2 = impl(q, k, v2, g, beta, S02, True)
    o3, s3 = impl(q, k, 2.0 * v - 3.0 * v2, g, beta, 2.0 * S0 - 3.0 * S02, True)
    np.testing.assert_allclose(o3, 2 * o1 - 3 * o2, atol=1e-12)
    np.testing.assert_allclose(s3, 2 * s1 - 3 * s2, atol=1e-12)
    v4 = v.copy(); v4[..., 2] = 7.0; S04 = S0.copy(); S04[..., 2] = -1.0
    o4, s4 = impl(q, k, v4, g, beta, S04, True)
    keep = [0, 1, 3, 4, 5]
    assert np.array_equal(o4[..., keep], o1[..., keep]) and np.array_equal(s4[..., keep], s1[..., keep])


def pin_resume(impl):
    """The state is all that carries over (fixed-size state): running [0,T) in one
    call equals [0,T1) then [T1,T) from the returned state, bitwise."""
    B, T, H, dk, dv, T1 = 2, 40, 2, 6, 5, 17
    q, k, v, g, beta = _rand(111, B, T, H, dk, dv)
    S0 = np.random.default_rng(112).standard_normal((B, H, dk, dv))
    o, S = impl(q, k, v, g, beta, S0, True)
    oa, Sa = impl(q[:, :T1], k[:, :T1], v[:, :T1], g[:, :T1], beta[:, :T1], S0, True)
    ob, Sb = impl(q[:, T1:], k[:, T1:], v[:, T1:], g[:, T1:], beta[:, T1:], Sa, True)
    assert np.array_equal(np.concatenate([oa, ob], axis=1), o) and np.array_equal(Sb, S)


def pin_bounded(impl):
    """With ||k|| <= 1, beta in [0,1] and alpha <= 1 every step is a contraction
    plus the write: ||S_t||_2 <= ||S_{t-1}||_2 + beta_t ||v_t||."""
    B, T, H, dk, dv = 1, 60, 1, 6, 6
    q, k, v, g, beta = _rand(121, B, T, H, dk, dv, gate_mu=-1.0)
    S = np.random.default_rng(122).standard_normal((B, H, dk, dv))
    for t in range(T):
        _, Sn = impl(q[:, t:t + 1], k[:, t:t + 1], v[:, t:t + 1], g[:, t:t + 1], beta[:, t:t + 1], S, True)
        lhs = np.linalg.norm(Sn[0, 0], 2)
        rhs = np.linalg.norm(S[0, 0], 2) + beta[0, t, 0] * np.linalg.norm(v[0, t, 0])
        assert lhs <= rhs * (1 + 1e-12)
        S = Sn


ALL_PINS = [pin_overwrite_narrative, pin_key_collision, pin_alpha_zero_clears,
            pin_alpha_zero_per_channel, pin_beta_zero, pin_additive_closed_form,
            pin_unit_key_self_recall, pin_orthonormal_recall, pin_kaczmarz_least_norm,
            pin_ogd_gradient, pin_decode_identity, pin_linearity_columns, pin_resume,
            pin_bounded]
