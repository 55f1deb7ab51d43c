"""Pins for the oracle's per-tensor current scaling (s = fl32(amax / 448), codes E4M3(fl32(x / s))).

TensorRT-LLM PR "TE FP8 attention backend for VisualGen": the Q/K/V and O scales are written
from the current tensors before every call. Pinned by a hand-computed case, the closed form at
power-of-two maxima (s exact, so the codes are the exact power-of-two rescaling), the largest
element encoding to +-448, power-of-two equivariance, the all-zero convention and the
dequantization error bound of a round-to-nearest E4M3 code.
"""
import numpy as np
import pytest

from oracle import current_quantize, current_scale, e4m3_decode, e4m3_encode


def test_hand_case():
    """amax 3: s = fl32(3/448). 1/s = 149.33 lies between the codes 144 (0x71, 1.125 * 2^7) and
    160 (0x72) and rounds to 144; -3/s = -448 is 0xFE; 0.5/s = 74.67 rounds to 72 (0x69,
    1.125 * 2^6), not 80."""
    codes, s = current_quantize(np.array([1.0, -3.0, 0.5], dtype=np.float32))
    assert s == np.float32(3.0) / np.float32(448.0)
    assert list(codes) == [0x71, 0xFE, 0x69]


def test_quotient_rounded_to_float32_before_the_code():
    """The codes are decided on the float32 quotient: amax 13 gives s = fl32(13/448), and the exact
    quotient -9.75 / s lies within half a float32 spacing (2^-16 at 336) of -336, so fl32(-9.75 / s)
    is -336 exactly, the midpoint of the E4M3 codes 320 (0x7A, even mantissa) and 352 (0x7B): the
    tie goes to 0xFA. Multiplying by the float32 reciprocal of s instead lands one float32 step
    past 336 and would give 0xFB."""
    from fractions import Fraction
    codes, s = current_quantize(np.array([13.0, -9.75], dtype=np.float32))
    assert s == np.float32(13.0) / np.float32(448.0)
    q = Fraction(-9.75) / Fraction(float(s))
    assert abs(q + 336) < Fraction(1, 2 ** 16)
    assert list(codes) == [0x7E, 0xFA]
    assert np.float32(np.float32(-9.75) * (np.float32(1.0) / s)) != np.float32(-336.0)


@pytest.mark.parametrize("k", [-20, -3, 0, 5, 30])
def test_power_of_two_maximum_closed_form(k):
    """amax = 448 * 2^k gives s = 2^k exactly, so the codes are E4M3(x * 2^-k)."""
    rng = np.random.default_rng(500 + k)
    x = (rng.standard_normal(1000) * 50).astype(np.float32) * np.float32(2.0 ** k)
    x = np.clip(x, -448 * 2.0 ** k, 448 * 2.0 ** k).astype(np.float32)
    x[17] = np.float32(-448 * 2.0 ** k)
    codes, s = current_quantize(x)
    assert s == np.float32(2.0 ** k)
    assert np.array_equal(codes, e4m3_encode(x.astype(np.float64) * 2.0 ** -k))


def test_largest_element_maps_to_448_and_equivariance():
    rng = np.random.default_rng(510)
    x = (rng.standard_normal((300, 3, 128)) * 7.3).astype(np.float32)
    codes, s = current_quantize(x)
    i = np.unravel_index(np.argmax(np.abs(x)), x.shape)
    assert codes[i] in (0x7E, 0xFE)
    assert np.all(np.abs(e4m3_decode(codes)) <= 448)
    for k in (-7, 4):   # scaling by 2^k scales s by 2^k and leaves the codes (no fp32 range limits here)
        c2, s2 = current_quantize((x * np.float32(2.0 ** k)).astype(np.float32))
        assert s2 == np.float32(s * np.float32(2.0 ** k)) and np.array_equal(c2, codes)


def test_all_zero_and_error_bound():
    codes, s = current_quantize(np.zeros((4, 2, 128), dtype=np.float32))
    assert s == 1.0 and np.all(codes == 0)
    rng = np.random.default_rng(511)
    x = (rng.standard_normal(20000) * np.exp2(rng.uniform(-12, 3, 20000))).astype(np.float32)
    codes, s = current_quantize(x)
    deq = e4m3_decode(codes) * np.float64(s)
    q = np.abs(x.astype(np.float64)) / np.float64(s)
    # half a code spacing at the quotient (normals: 2^-4 relative; subnormals: 2^-10 absolute),
    # plus the float32 rounding of the quotient itself
    step = np.where(q >= 2.0 ** -6, np.exp2(np.floor(np.log2(np.maximum(q, 2.0 ** -6))) - 3), 2.0 ** -9)
    assert np.all(np.abs(deq - x) <= (0.5 * step + q * 2.0 ** -23) * np.float64(s) * (1 + 1e-9))
    assert current_scale(np.array([2.0, -8.0], dtype=np.float32)) == np.float32(8.0) / np.float32(448.0)
