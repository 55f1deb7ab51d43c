"""CPU check of the element-wise rounding bound the GPU parity tests use for E4M3 and BF16
probabilities (helpers.pv_rounding_bound).

A NumPy model of what the kernel may do within its contract rounds each probability against
its own reference maximum (a running maximum up to 2^8 below the final one, chosen per key,
so lambda_j = 2^(m - m_j) ranges over [1, 256]) and normalises by the sum of its rounded
probabilities. Its distance from the oracle's output must stay inside the bound on inputs
with x20 outliers, for both probability types; a model that drops a key must not.
"""
import numpy as np
import pytest
import torch

import oracle
from helpers import pv_rounding_bound
from synth import make_custom, bf16_bits_to_f32


def _round(x, mode):
    dt = torch.bfloat16 if mode == "bf16" else torch.float8_e4m3fn
    return torch.from_numpy(x.astype(np.float32)).to(dt).to(torch.float64).numpy()


def _model(qhat, khat, v, cu, mode, rng, drop=False):
    tq, h, d = qhat.shape
    out = np.zeros_like(qhat)
    for r in range(len(cu) - 1):
        a, b = cu[r], cu[r + 1]
        for hh in range(h):
            s = (qhat[a:b, hh] @ khat[a:b, hh].T) / np.sqrt(d)
            p = np.exp(s - s.max(axis=1, keepdims=True))
            lam = np.exp2(rng.uniform(0.0, 8.0, p.shape))
            lam = np.minimum(lam, 256.0 / np.maximum(p, 1e-300))    # the kernel's P stays <= 2^8
            q = _round(p * lam, mode) / lam
            if drop:
                q[:, -1] = 0.0
            out[a:b, hh] = (q @ v[a:b, hh]) / q.sum(axis=1, keepdims=True)
    return _round(out, "bf16")


@pytest.mark.parametrize("mode", ["fp8", "bf16"])
def test_bound_covers_the_model(mode):
    rng = np.random.default_rng(900)
    wl = make_custom([300, 77], [300, 77], heads=2, seed=901, outlier_rate=2e-3)
    f = lambda bits: bf16_bits_to_f32(bits).astype(np.float64)
    pq, sq, cs = oracle.mx_quantize_varlen(f(wl.q_bits), wl.cu_q)
    pk, sk, _ = oracle.mx_quantize_varlen(f(wl.k_bits), wl.cu_k)
    qh, kh = oracle.mx_dequantize_varlen(pq, sq, wl.cu_q, cs), oracle.mx_dequantize_varlen(pk, sk, wl.cu_k, cs)
    v = oracle.e4m3_decode(oracle.e4m3_cast(f(wl.v_bits))) if mode == "fp8" else f(wl.v_bits)
    ref = oracle.attention_varlen(qh, kh, v, wl.cu_q, wl.cu_k, pv_mode=mode)
    rows = {0: np.arange(300), 1: np.arange(77)}
    bound = pv_rounding_bound(qh, kh, v, wl.cu_q, wl.cu_k, rows, mode, ref)
    got = _model(qh, kh, v, wl.cu_q, mode, rng)
    err = np.abs(got - ref.out)
    assert np.all(err <= bound), float((err / bound).max())
    assert np.max(err / bound) > 0.01          # the bound is not vacuous on this data
    bad = _model(qh, kh, v, wl.cu_q, mode, rng, drop=True)
    assert np.any(np.abs(bad - ref.out) > bound)
