"""Pins for the oracle's attention backward (oracle/backward.py), independent of its own formulas.

* Central finite differences of the forward loss sum(dO * O), with O = softmax(tau Q K^T) V in
  float64, give dQ, dK and dV (every term, sign and transposition of the backward).
* Closed forms: one key (P = 1: dQ = dK = 0, dV = sum of dO); Q = 0 (uniform P: dV_j = mean dO).
* Invariance: shifting every key by one vector leaves all three gradients unchanged, because
  each row of dS sums to zero when D is taken from the exact output.
* Orientation routing: dK is linear in Q's token orientation and nothing else depends on it;
  the same for dQ and K's token orientation; dV does not depend on V.
* Packed sequences equal each sequence alone; the BF16 operand rounding stays within its
  relative bound.
"""
import numpy as np
import pytest

import oracle


def _forward(q, k, v, cu_q, cu_k, tau):
    """Plain float64 forward: O and the natural-log LSE of the scaled scores."""
    tq, h, d = q.shape
    out = np.zeros_like(q)
    lse = np.zeros((h, tq))
    for r in range(len(cu_q) - 1):
        q0, q1, k0, k1 = cu_q[r], cu_q[r + 1], cu_k[r], cu_k[r + 1]
        for hh in range(h):
            s = tau * (q[q0:q1, hh] @ k[k0:k1, hh].T)
            m = s.max(axis=1, keepdims=True)
            u = np.exp(s - m)
            l = u.sum(axis=1, keepdims=True)
            out[q0:q1, hh] = (u / l) @ v[k0:k1, hh]
            lse[hh, q0:q1] = (m + np.log(l))[:, 0]
    return out, lse


def _problem(seed, lq=(3, 4), lk=(5, 2), h=2, d=16, scale=1.0):
    rng = np.random.default_rng(seed)
    cu_q = np.concatenate([[0], np.cumsum(lq)]).astype(np.int64)
    cu_k = np.concatenate([[0], np.cumsum(lk)]).astype(np.int64)
    q = rng.standard_normal((cu_q[-1], h, d)) * scale
    k = rng.standard_normal((cu_k[-1], h, d)) * scale
    v = rng.standard_normal((cu_k[-1], h, d))
    do = rng.standard_normal((cu_q[-1], h, d))
    return q, k, v, do, cu_q, cu_k


def _exact_bwd(q, k, v, do, cu_q, cu_k, tau, qt=None, kt=None, round_ops="none"):
    out, lse = _forward(q, k, v, cu_q, cu_k, tau)
    return oracle.attention_varlen_bwd(q, k, v, q if qt is None else qt, k if kt is None else kt,
                                       out, do, lse, cu_q, cu_k, softmax_scale=tau,
                                       round_ops=round_ops)


def test_finite_differences():
    q, k, v, do, cu_q, cu_k = _problem(700)
    tau = 0.3
    g = _exact_bwd(q, k, v, do, cu_q, cu_k, tau)

    def loss(q_, k_, v_):
        return float(np.sum(do * _forward(q_, k_, v_, cu_q, cu_k, tau)[0]))

    eps = 1e-6
    for name, x, grad in (("q", q, g.dq), ("k", k, g.dk), ("v", v, g.dv)):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += eps
            xm[idx] -= eps
            args_p = {"q": (xp, k, v), "k": (q, xp, v), "v": (q, k, xp)}[name]
            args_m = {"q": (xm, k, v), "k": (q, xm, v), "v": (q, k, xm)}[name]
            num[idx] = (loss(*args_p) - loss(*args_m)) / (2 * eps)
        np.testing.assert_allclose(grad, num, rtol=1e-6, atol=1e-8, err_msg=name)


def test_single_key_closed_form():
    q, k, v, do, cu_q, cu_k = _problem(701, lq=(6,), lk=(1,))
    g = _exact_bwd(q, k, v, do, cu_q, cu_k, 0.25)
    assert np.max(np.abs(g.dq)) < 1e-12 and np.max(np.abs(g.dk)) < 1e-12
    np.testing.assert_allclose(g.dv[0], do.sum(axis=0), rtol=1e-13, atol=1e-13)


def test_zero_queries_closed_form():
    q, k, v, do, cu_q, cu_k = _problem(702, lq=(5,), lk=(8,))
    q[:] = 0.0
    g = _exact_bwd(q, k, v, do, cu_q, cu_k, 0.25, round_ops="bf16")  # P = 1/8 is exact in BF16
    np.testing.assert_allclose(g.dv, np.broadcast_to(do.sum(axis=0) / 8, g.dv.shape), rtol=1e-13, atol=1e-13)
    assert np.max(np.abs(g.dk)) == 0.0  # Q's token orientation is zero too


def test_key_shift_invariance():
    q, k, v, do, cu_q, cu_k = _problem(703)
    tau = 0.4
    c = np.random.default_rng(1).standard_normal(k.shape[1:])  # one vector per head
    g0 = _exact_bwd(q, k, v, do, cu_q, cu_k, tau)
    g1 = _exact_bwd(q, k + c[None], v, do, cu_q, cu_k, tau)
    for a, b in ((g0.dq, g1.dq), (g0.dk, g1.dk), (g0.dv, g1.dv)):
        np.testing.assert_allclose(a, b, rtol=1e-9, atol=1e-11)


def test_orientation_routing():
    q, k, v, do, cu_q, cu_k = _problem(704)
    tau = 0.3
    rng = np.random.default_rng(2)
    qt, kt = rng.standard_normal(q.shape), rng.standard_normal(k.shape)
    base = _exact_bwd(q, k, v, do, cu_q, cu_k, tau, qt=qt, kt=kt, round_ops="bf16")
    q2 = _exact_bwd(q, k, v, do, cu_q, cu_k, tau, qt=2 * qt, kt=kt, round_ops="bf16")
    k2 = _exact_bwd(q, k, v, do, cu_q, cu_k, tau, qt=qt, kt=2 * kt, round_ops="bf16")
    assert np.array_equal(q2.dk, 2 * base.dk) and np.array_equal(q2.dq, base.dq) and np.array_equal(q2.dv, base.dv)
    assert np.array_equal(k2.dq, 2 * base.dq) and np.array_equal(k2.dk, base.dk) and np.array_equal(k2.dv, base.dv)
    # dV = P^T dO does not involve V (the output passed in stays the same)
    out, lse = _forward(q, k, v, cu_q, cu_k, tau)
    g_a = oracle.attention_varlen_bwd(q, k, v, qt, kt, out, do, lse, cu_q, cu_k, tau)
    g_b = oracle.attention_varlen_bwd(q, k, 3 * v, qt, kt, out, do, lse, cu_q, cu_k, tau)
    assert np.array_equal(g_a.dv, g_b.dv) and not np.allclose(g_a.dq, g_b.dq)


def test_packed_equals_each_sequence():
    q, k, v, do, cu_q, cu_k = _problem(705, lq=(4, 0, 3), lk=(2, 3, 6))
    tau = 0.3
    g = _exact_bwd(q, k, v, do, cu_q, cu_k, tau, round_ops="bf16")
    for r in range(3):
        qs, ks = slice(cu_q[r], cu_q[r + 1]), slice(cu_k[r], cu_k[r + 1])
        one = _exact_bwd(q[qs], k[ks], v[ks], do[qs], [0, cu_q[r + 1] - cu_q[r]],
                         [0, cu_k[r + 1] - cu_k[r]], tau, round_ops="bf16")
        assert np.array_equal(one.dq, g.dq[qs]) and np.array_equal(one.dk, g.dk[ks])
        assert np.array_equal(one.dv, g.dv[ks])
    assert np.all(g.dk[cu_k[1]:cu_k[2]] == 0) and np.all(g.dv[cu_k[1]:cu_k[2]] == 0)  # no queries


def test_bf16_operand_rounding_bound():
    q, k, v, do, cu_q, cu_k = _problem(706, lq=(40,), lk=(70,), d=32)
    tau = 0.2
    exact = _exact_bwd(q, k, v, do, cu_q, cu_k, tau)
    rnd = _exact_bwd(q, k, v, do, cu_q, cu_k, tau, round_ops="bf16")
    out, lse = _forward(q, k, v, cu_q, cu_k, tau)
    # |r(x) - x| <= 2^-8 |x| for BF16 round to nearest: bound each sum by the sum of magnitudes
    for hh in range(q.shape[1]):
        s = tau * q[:, hh] @ k[:, hh].T
        p = np.exp(s - lse[hh][:, None])
        ds = p * (do[:, hh] @ v[:, hh].T - np.sum(do[:, hh] * out[:, hh], axis=1)[:, None])
        bound_v = 2.0 ** -8 * (p.T @ np.abs(do[:, hh])) + 1e-13
        bound_k = 2.0 ** -8 * tau * (np.abs(ds).T @ np.abs(q[:, hh])) + 1e-13
        bound_q = 2.0 ** -8 * tau * (np.abs(ds) @ np.abs(k[:, hh])) + 1e-13
        assert np.all(np.abs(rnd.dv[:, hh] - exact.dv[:, hh]) <= bound_v)
        assert np.all(np.abs(rnd.dk[:, hh] - exact.dk[:, hh]) <= bound_k)
        assert np.all(np.abs(rnd.dq[:, hh] - exact.dq[:, hh]) <= bound_q)
    assert not np.array_equal(rnd.dv, exact.dv)


def test_queries_without_keys_rejected():
    q, k, v, do, cu_q, cu_k = _problem(707, lq=(3, 2), lk=(4, 0))
    out = np.zeros_like(q)
    with pytest.raises(ValueError):
        oracle.attention_varlen_bwd(q, k, v, q, k, out, do, np.zeros((2, 5)), cu_q, cu_k)
