"""Pins for the oracle's attention: brute force on tiny shapes, closed forms, varlen and descale invariants.

The brute force here is a second, independent implementation in plain Python
(math.fsum sums, math.exp) that rounds the probabilities with torch's own CPU
casts (bfloat16 / float8_e4m3fn), so it shares no arithmetic with the oracle.
Shapes use Sq != Sk and non-symmetric data so that a transposed operand, a
dropped softmax scale, a wrong normaliser or a mixed-up sequence shows up.
"""
import math

import numpy as np
import pytest
import torch

from oracle import attention_varlen, e4m3_decode, e4m3_cast

D = 128


def _torch_round(u: float, mode: str) -> float:
    dt = torch.bfloat16 if mode == "bf16" else torch.float8_e4m3fn
    return float(torch.tensor([u], dtype=torch.float32).to(dt).to(torch.float64)[0])


def _brute(q, k, v, cu_q, cu_k, mode, scale, qd=None, kd=None, vd=None):
    tq, h, d = q.shape
    out = np.zeros((tq, h, d))
    lse = np.zeros((h, tq))
    for r in range(len(cu_q) - 1):
        for hh in range(h):
            c = scale * (1.0 if qd is None else qd[r][hh]) * (1.0 if kd is None else kd[r][hh])
            vv = 1.0 if vd is None else vd[r][hh]
            keys = range(cu_k[r], cu_k[r + 1])
            for i in range(cu_q[r], cu_q[r + 1]):
                s = [c * math.fsum(float(q[i, hh, t]) * float(k[j, hh, t]) for t in range(d)) for j in keys]
                m = max(s)
                u = [math.exp(x - m) for x in s]
                l = math.fsum(u)
                p = [_torch_round(x, mode) for x in u]
                for t in range(d):
                    out[i, hh, t] = vv * math.fsum(pj * float(v[j, hh, t]) for pj, j in zip(p, keys)) / l
                lse[hh, i] = m + math.log(l)
    return out, lse


def _fp8_values(rng, shape, spread=4):
    """Random E4M3-representable values times per-row powers of two (like dequantized MX operands)."""
    codes = rng.integers(0, 0x7F, size=shape)
    codes = np.where(codes == 0x7F, 0x7E, codes) | (rng.integers(0, 2, size=shape) << 7)
    vals = e4m3_decode(codes.astype(np.uint8)) * 2.0 ** -6
    return vals * np.exp2(rng.integers(-spread, spread + 1, size=shape[:2] + (1,)))


@pytest.mark.parametrize("mode", ["bf16", "fp8"])
def test_brute_force_tiny(mode):
    rng = np.random.default_rng(21)
    cu_q, cu_k = [0, 3, 8], [0, 5, 7]                  # two sequences, Lq != Lk
    q = _fp8_values(rng, (8, 2, D))
    k = _fp8_values(rng, (7, 2, D))
    v = rng.standard_normal((7, 2, D))
    if mode == "fp8":
        v = e4m3_decode(e4m3_cast(v))
    else:
        v = np.asarray(torch.tensor(v).to(torch.bfloat16).to(torch.float64))
    scale = 1 / math.sqrt(D)
    ref_o, ref_l = _brute(q, k, v, cu_q, cu_k, mode, scale)
    res = attention_varlen(q, k, v, cu_q, cu_k, pv_mode=mode)
    np.testing.assert_allclose(res.out, ref_o, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(res.lse, ref_l, rtol=1e-12, atol=1e-13)


def test_brute_force_descales():
    rng = np.random.default_rng(22)
    cu = [0, 4, 6]
    q = _fp8_values(rng, (6, 2, D))
    k = _fp8_values(rng, (6, 2, D))
    v = e4m3_decode(e4m3_cast(rng.standard_normal((6, 2, D))))
    qd, kd, vd = (np.exp2(rng.uniform(-4, 2, (2, 2))) for _ in range(3))
    ref_o, ref_l = _brute(q, k, v, cu, cu, "fp8", 1 / math.sqrt(D), qd, kd, vd)
    res = attention_varlen(q, k, v, cu, cu, pv_mode="fp8", q_descale=qd, k_descale=kd, v_descale=vd)
    np.testing.assert_allclose(res.out, ref_o, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(res.lse, ref_l, rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("mode", ["bf16", "fp8"])
def test_zero_queries_closed_form(mode):
    """Q = 0: every score is 0, every probability rounds to exactly 1: O = mean_j V'_j, LSE = ln Sk."""
    rng = np.random.default_rng(23)
    sk = 37
    q = np.zeros((5, 3, D))
    k = rng.standard_normal((sk, 3, D))
    v = rng.standard_normal((sk, 3, D))
    res = attention_varlen(q, k, v, [0, 5], [0, sk], pv_mode=mode)
    np.testing.assert_allclose(res.out, np.broadcast_to(v.mean(axis=0), (5, 3, D)), rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(res.lse, math.log(sk), rtol=1e-14)


def test_single_key_closed_form():
    """Sk = 1: O = V'_0 and LSE = the one scaled score."""
    rng = np.random.default_rng(24)
    q = rng.standard_normal((4, 2, D))
    k = rng.standard_normal((1, 2, D))
    v = rng.standard_normal((1, 2, D))
    res = attention_varlen(q, k, v, [0, 4], [0, 1], pv_mode="bf16", softmax_scale=0.3)
    np.testing.assert_allclose(res.out, np.broadcast_to(v[0], (4, 2, D)), rtol=1e-14)
    expect = 0.3 * np.einsum("thd,hd->ht", q, k[0])
    np.testing.assert_allclose(res.lse, expect, rtol=1e-13)


@pytest.mark.parametrize("mode,tol", [("bf16", 2.0 ** -8), ("fp8", 2.0 ** -3)])
def test_constant_values_normalisation(mode, tol):
    """V = 1: O = sum(P~)/sum(u) = 1 within the probability rounding's relative error."""
    rng = np.random.default_rng(25)
    q = rng.standard_normal((50, 2, D))
    k = rng.standard_normal((300, 2, D))
    v = np.ones((300, 2, D))
    res = attention_varlen(q, k, v, [0, 50], [0, 300], pv_mode=mode)
    assert np.all(np.abs(res.out - 1.0) <= tol)


def test_softmax_rows_sum_to_one():
    """With the rounding removed (a V of identity columns), the weights sum to 1 to 1e-12."""
    rng = np.random.default_rng(26)
    sk = 128
    q = rng.standard_normal((20, 1, D))
    k = rng.standard_normal((sk, 1, D))
    # V'_j = e_j (one-hot rows): O_i[j] = P~_ij / l_i; use bf16 mode and compare to exp-normalised scores
    v = np.eye(sk)[:, None, :]
    res = attention_varlen(q, k, v, [0, 20], [0, sk], pv_mode="bf16")
    s = (q[:, 0] @ k[:, 0].T) / math.sqrt(D)
    w = np.exp(s - s.max(axis=1, keepdims=True))
    w /= w.sum(axis=1, keepdims=True)
    assert np.all(np.abs(w.sum(axis=1) - 1) < 1e-12)
    np.testing.assert_allclose(res.out[:, 0], w, rtol=2.0 ** -8, atol=1e-30)


def test_packed_varlen_equals_per_sequence():
    rng = np.random.default_rng(27)
    lq, lk = [7, 1, 30, 0, 12], [9, 40, 3, 5, 12]
    cu_q, cu_k = np.concatenate([[0], np.cumsum(lq)]), np.concatenate([[0], np.cumsum(lk)])
    q = rng.standard_normal((cu_q[-1], 2, D))
    k = rng.standard_normal((cu_k[-1], 2, D))
    v = rng.standard_normal((cu_k[-1], 2, D))
    packed = attention_varlen(q, k, v, cu_q, cu_k, pv_mode="fp8")
    for r in range(len(lq)):
        if lq[r] == 0:
            continue
        a, b, c, d = cu_q[r], cu_q[r + 1], cu_k[r], cu_k[r + 1]
        alone = attention_varlen(q[a:b], k[c:d], v[c:d], [0, b - a], [0, d - c], pv_mode="fp8")
        assert np.array_equal(alone.out, packed.out[a:b])
        assert np.array_equal(alone.lse, packed.lse[:, a:b])


def test_unit_descale_is_exact_and_two_changes_output():
    rng = np.random.default_rng(28)
    q = rng.standard_normal((16, 2, D))
    k = rng.standard_normal((16, 2, D))
    v = rng.standard_normal((16, 2, D))
    none = attention_varlen(q, k, v, [0, 16], [0, 16], pv_mode="fp8")
    ones = np.ones((1, 2))
    unit = attention_varlen(q, k, v, [0, 16], [0, 16], pv_mode="fp8",
                            q_descale=ones, k_descale=ones, v_descale=ones)
    assert np.array_equal(none.out, unit.out) and np.array_equal(none.lse, unit.lse)
    two = attention_varlen(q, k, v, [0, 16], [0, 16], pv_mode="fp8", q_descale=2 * ones)
    assert not np.array_equal(none.out, two.out)
    assert not np.array_equal(none.lse, two.lse)


def test_row_subset_matches_full():
    rng = np.random.default_rng(29)
    q = rng.standard_normal((100, 2, D))
    k = rng.standard_normal((80, 2, D))
    v = rng.standard_normal((80, 2, D))
    full = attention_varlen(q, k, v, [0, 60, 100], [0, 50, 80], pv_mode="bf16", row_block=7)
    sub = attention_varlen(q, k, v, [0, 60, 100], [0, 50, 80], pv_mode="bf16",
                           rows={0: np.array([0, 13, 59]), 1: np.array([39])})
    for i in (0, 13, 59, 99):
        # same values up to float64 rounding (BLAS blocking depends on the matrix shape)
        np.testing.assert_allclose(sub.out[i], full.out[i], rtol=1e-13, atol=1e-15)
        np.testing.assert_allclose(sub.lse[:, i], full.lse[:, i], rtol=1e-14)
    assert np.isnan(sub.out[1]).all()


def test_keys_without_queries_rejected():
    q = np.zeros((2, 1, D))
    with pytest.raises(ValueError):
        attention_varlen(q, np.zeros((0, 1, D)), np.zeros((0, 1, D)), [0, 2], [0, 0])
