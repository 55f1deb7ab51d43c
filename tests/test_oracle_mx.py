"""Pins for the oracle's MXFP8 quantizer: hand-computed block encodings, invariants, scale layout.

Hand cases live in tests/golden/mx_block_cases.json with their derivations. The
invariants follow from the RCEIL/FLOOR readings (the LP-FA4 README names the
modes only): power-of-two equivariance, the range of the block maximum's code,
the dequantization error bound of a round-to-nearest E4M3 code, and the
per-sequence 128-token-padded scale layout with 0x7F pad rows.
"""
import json
import os

import numpy as np
import pytest

from oracle import (e4m3_decode, mx_block_exponent, mx_quantize_varlen, mx_dequantize_varlen,
                    padded_len, scale_offsets, e4m3_cast, pertensor_quantize, e4m3_encode)
from synth import make_custom, bf16_bits_to_f32

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "mx_block_cases.json")


def _block_with_max(amax, rng):
    """A 32-element block whose largest magnitude is amax, at a random position, other entries smaller."""
    blk = rng.uniform(-1.0, 1.0, 32) * amax * 0.5
    pos = int(rng.integers(0, 32))
    blk[pos] = amax if rng.random() < 0.5 else -amax
    return blk, pos


@pytest.mark.parametrize("mode", ["rceil", "floor"])
def test_golden_block_cases(mode):
    cases = json.load(open(GOLDEN))["cases"]
    rng = np.random.default_rng(11)
    for c in cases:
        blk, pos = _block_with_max(c["amax"], rng)
        x = np.zeros((1, 1, 128))
        x[0, 0, 32:64] = blk             # second block of the row
        payload, scales, _ = mx_quantize_varlen(x, np.array([0, 1]), mode)
        assert int(scales[0, 0, 1]) == c[f"{mode}_byte"], c
        assert int(payload[0, 0, 32 + pos]) & 0x7F == c[f"{mode}_payload"], c
        # the other (all-zero) blocks take the zero-block encoding
        assert int(scales[0, 0, 0]) == 0 and np.all(payload[0, 0, :32] == 0)


def test_rceil_and_floor_relation():
    """FLOOR's exponent is RCEIL's or one less; they agree exactly when amax has mantissa <= 1.75."""
    rng = np.random.default_rng(5)
    amax = np.abs(rng.standard_normal(20000)) * np.exp2(rng.integers(-100, 100, 20000))
    er = mx_block_exponent(amax, "rceil")
    ef = mx_block_exponent(amax, "floor")
    mant = amax / np.exp2(np.floor(np.log2(amax)))
    assert np.all((er - ef == 0) | (er - ef == 1))
    assert np.array_equal(er - ef == 1, mant > 1.75)


def _rand_tensor(rng, t, h, spread=True):
    x = rng.standard_normal((t, h, 128))
    if spread:
        x *= np.exp2(rng.integers(-20, 20, (t, h, 4)).repeat(32, axis=2))
    return x


def test_rceil_invariants():
    rng = np.random.default_rng(1)
    x = _rand_tensor(rng, 40, 3)
    payload, scales, _ = mx_quantize_varlen(x, np.array([0, 40]), "rceil")
    vals = np.abs(e4m3_decode(payload)).reshape(40, 3, 4, 32)
    assert np.all(vals <= 448)
    top = vals.max(axis=3)
    assert np.all((top >= 224) & (top <= 448))       # rounded block maximum lands in [224, 448]
    e = scales[:40].astype(np.int64) - 127
    pre = np.abs(x.reshape(40, 3, 4, 32)).max(axis=3) * np.exp2(-e.astype(np.float64))
    assert np.all((pre > 224) & (pre <= 448))        # before rounding: (224, 448]


def test_floor_invariant_before_saturation():
    rng = np.random.default_rng(2)
    x = _rand_tensor(rng, 40, 3)
    payload, scales, _ = mx_quantize_varlen(x, np.array([0, 40]), "floor")
    e = scales[:40].astype(np.int64) - 127
    blocks = x.reshape(40, 3, 4, 32)
    pre = np.abs(blocks).max(axis=3) * np.exp2(-e.astype(np.float64))
    assert np.all((pre >= 256) & (pre < 512))


@pytest.mark.parametrize("mode", ["rceil", "floor"])
def test_power_of_two_equivariance(mode):
    rng = np.random.default_rng(3)
    x = _rand_tensor(rng, 16, 2, spread=False)
    p0, s0, _ = mx_quantize_varlen(x, np.array([0, 16]), mode)
    for k in (-30, -1, 1, 7, 50):
        pk, sk, _ = mx_quantize_varlen(x * 2.0 ** k, np.array([0, 16]), mode)
        assert np.array_equal(pk, p0)
        assert np.array_equal(sk[:16].astype(int), s0[:16].astype(int) + k)


@pytest.mark.parametrize("mode", ["rceil", "floor"])
def test_dequant_error_bound(mode):
    """|x - deq(q(x))| <= half an E4M3 step at the block's scale (2^-4 relative for normals,
    2^-10 * 2^e absolute in the subnormal range), except FLOOR's saturated maxima (<= 64 * 2^e)."""
    rng = np.random.default_rng(4)
    x = _rand_tensor(rng, 30, 2)
    payload, scales, cu_scale = mx_quantize_varlen(x, np.array([0, 30]), mode)
    deq = mx_dequantize_varlen(payload, scales, np.array([0, 30]), cu_scale)
    e = (scales[:30].astype(np.float64) - 127).repeat(32, axis=2)
    unit = np.exp2(e)
    bound = np.maximum(np.abs(x) * 2.0 ** -4, 2.0 ** -10 * unit)
    if mode == "floor":
        bound = np.maximum(bound, np.where(np.abs(x) / unit > 448, 64 * unit, 0))
    assert np.all(np.abs(deq - x) <= bound * (1 + 1e-12))


def test_scale_layout_and_padding():
    lengths = [5, 128, 129, 0, 300]
    wl = make_custom(lengths, lengths, heads=3, seed=9)
    x = bf16_bits_to_f32(wl.q_bits).astype(np.float64)
    cu = wl.cu_q
    payload, scales, cu_scale = mx_quantize_varlen(x, cu, "rceil")
    assert list(cu_scale) == [0, 128, 256, 512, 512, 896]
    assert [padded_len(v) for v in lengths] == [128, 128, 256, 0, 384]
    assert np.array_equal(cu_scale, scale_offsets(lengths))
    assert scales.shape == (896, 3, 4)
    for i, length in enumerate(lengths):
        s0 = int(cu_scale[i])
        pad = scales[s0 + length:int(cu_scale[i + 1])]
        assert np.all(pad == 0x7F)
        # each sequence quantized alone gives the same bytes (per-token blocks, per-sequence storage)
        c0 = int(cu[i])
        pi, si, _ = mx_quantize_varlen(x[c0:c0 + length], np.array([0, length]), "rceil")
        assert np.array_equal(pi, payload[c0:c0 + length])
        assert np.array_equal(si[:length], scales[s0:s0 + length])


def test_bf16_and_fp32_inputs_agree_on_bf16_values():
    """A BF16 tensor widened to FP32 is the same set of values: identical bytes."""
    wl = make_custom([64], [64], heads=2, seed=10)
    x32 = bf16_bits_to_f32(wl.q_bits)
    a = mx_quantize_varlen(x32.astype(np.float64), np.array([0, 64]))
    b = mx_quantize_varlen(x32, np.array([0, 64]))
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_e4m3_cast_and_pertensor():
    x = np.array([[[1.0, -500.0, 2.0 ** -11, 3.3]]])
    assert list(e4m3_cast(x).ravel()) == [0x38, 0xFE, 0x00, 0x45]   # 3.3 -> 3.25 = 1.625*2
    # per-tensor: E4M3(x / s); a power-of-two s just shifts the exponent field
    x = np.full((4, 2, 128), 1.5)
    d = np.array([[0.125, 1.0]])
    p = pertensor_quantize(x, np.array([0, 4]), d)
    assert np.all(p[:, 0] == e4m3_encode(np.array([12.0]))[0]) and np.all(p[:, 1] == 0x3C)
    assert np.array_equal(pertensor_quantize(x, np.array([0, 4]), None), e4m3_encode(x))
