"""Pins for the oracle's number formats (E4M3, E8M0, BF16) against closed forms and torch's CPU casts.

The E4M3 encoder is checked three independent ways: values computed by hand from
the OCP E4M3FN field definition, a brute-force nearest search written here in
plain Python, and torch's own float8_e4m3fn CPU cast (a library routine, not the
oracle) over every BF16 value of magnitude at most 464 (above 464 torch returns
NaN where the saturating reading gives 448).
"""
import math
import struct

import numpy as np
import pytest
import torch

from oracle import e4m3_decode, e4m3_encode, e8m0_decode, bf16_round, bf16_encode, E4M3_VALUES


def test_e4m3_decode_closed_forms():
    assert e4m3_decode(np.array([0x7E]))[0] == 448.0
    assert e4m3_decode(np.array([0xFE]))[0] == -448.0
    assert e4m3_decode(np.array([0x38]))[0] == 1.0
    assert e4m3_decode(np.array([0x01]))[0] == 2.0 ** -9          # smallest subnormal
    assert e4m3_decode(np.array([0x07]))[0] == 7 * 2.0 ** -9       # largest subnormal
    assert e4m3_decode(np.array([0x08]))[0] == 2.0 ** -6           # smallest normal
    assert e4m3_decode(np.array([0x70]))[0] == 128.0
    assert e4m3_decode(np.array([0x3C]))[0] == 1.5
    assert math.isnan(e4m3_decode(np.array([0x7F]))[0])
    assert math.isnan(e4m3_decode(np.array([0xFF]))[0])
    z = e4m3_decode(np.array([0x80]))[0]
    assert z == 0.0 and math.copysign(1.0, z) == -1.0
    # 126 positive finite codes above zero, strictly increasing; negatives mirror positives
    pos = E4M3_VALUES[:0x7F]
    assert np.all(np.diff(pos) > 0)
    assert np.array_equal(E4M3_VALUES[0x80:0xFF], -pos)


def test_e4m3_decode_matches_torch_bit_reinterpretation():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ours = e4m3_decode(np.arange(256))
    both_nan = np.isnan(ref) & np.isnan(ours)
    assert np.all(both_nan | (ref == ours))


HAND = [  # value -> code, worked out from the field definition (nearest, ties to even, saturate)
    (448.0, 0x7E), (464.0, 0x7E), (1e6, 0x7E), (-1e6, 0xFE), (250.0, 0x78), (300.0, 0x79),
    (240.0, 0x77), (2.0 ** -10, 0x00), (3 * 2.0 ** -10, 0x02), (0.001, 0x01), (-(2.0 ** -11), 0x80),
    (1.0, 0x38), (-0.0, 0x80), (0.0, 0x00), (432.0, 0x7E), (431.9, 0x7D), (0.0146484375, 0x08),
    (1.0625, 0x38), (1.1875, 0x3A), (17.0, 0x58), (-17.0, 0xD8), (19.0, 0x5A), (2.0 ** -9 * 1.5, 0x02),
]


@pytest.mark.parametrize("x,code", HAND)
def test_e4m3_encode_hand_values(x, code):
    assert int(e4m3_encode(np.array([x]))[0]) == code


def _brute_nearest(x: float) -> int:
    """Nearest finite code by scanning all 254 finite codes; ties to the even code; saturate."""
    best, best_d = None, None
    for c in range(256):
        if (c & 0x7F) == 0x7F:
            continue
        v = float(E4M3_VALUES[c])
        if (c & 0x80) != (0x80 if math.copysign(1.0, x) < 0 else 0):
            continue
        d = abs(v - x)
        if best is None or d < best_d or (d == best_d and c % 2 == 0):
            best, best_d = c, d
    return best


def test_e4m3_encode_vs_brute_force():
    rng = np.random.default_rng(7)
    xs = np.concatenate([rng.standard_normal(600) * 30, rng.standard_normal(300) * 0.01,
                         rng.uniform(-500, 500, 200), (np.arange(-60, 61) / 8.0) ** 3])
    got = e4m3_encode(xs)
    for x, g in zip(xs, got):
        assert int(g) == _brute_nearest(float(x)), x


def _all_bf16_values():
    bits = np.arange(65536, dtype=np.uint32) << 16
    f = bits.view(np.float32)
    return f[np.isfinite(f)]


def test_e4m3_encode_vs_torch_all_bf16():
    f = _all_bf16_values()
    f = f[np.abs(f) <= 464.0]
    ref = torch.from_numpy(f.copy()).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    ours = e4m3_encode(f.astype(np.float64))
    assert np.array_equal(ours, ref)


def test_e4m3_encode_saturates_above_464():
    f = _all_bf16_values()
    big = f[np.abs(f) > 464.0].astype(np.float64)
    codes = e4m3_encode(big)
    assert np.all((codes & 0x7F) == 0x7E)
    assert np.array_equal(codes >> 7, (big < 0).astype(np.uint8))


def test_e8m0_decode():
    assert e8m0_decode(np.array([127]))[0] == 1.0
    assert e8m0_decode(np.array([0]))[0] == 2.0 ** -127
    assert e8m0_decode(np.array([254]))[0] == 2.0 ** 127
    assert e8m0_decode(np.array([128]))[0] == 2.0
    with pytest.raises(ValueError):
        e8m0_decode(np.array([255]))


def test_bf16_round_vs_torch():
    rng = np.random.default_rng(3)
    bits = rng.integers(0, 2 ** 32, size=200000, dtype=np.uint64).astype(np.uint32)
    f = bits.view(np.float32)
    f = f[np.isfinite(f) & (np.abs(f) < 3.0e38)]
    f = np.concatenate([f, np.float32([1.00390625, 1.01171875, 1.0, 0.0, -0.0, 1e-40, -3e-39])])
    ref = torch.from_numpy(f.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    ours = bf16_encode(f.astype(np.float64))
    assert np.array_equal(ours, ref)


def test_bf16_round_hand_values():
    # 1 + 2^-8 is halfway between 1 and 1 + 2^-7: ties to even -> 1
    assert bf16_round(np.array([1.0 + 2.0 ** -8]))[0] == 1.0
    # 1 + 3*2^-8 is halfway between 1 + 2^-7 and 1 + 2^-6: even mantissa is 1 + 2^-6
    assert bf16_round(np.array([1.0 + 3 * 2.0 ** -8]))[0] == 1.0 + 2.0 ** -6
    assert bf16_round(np.array([0.3]))[0] == struct.unpack(">f", bytes.fromhex("3e9a0000"))[0]
    assert bf16_round(np.array([2.0 ** -140]))[0] == 0.0               # below half the smallest subnormal
    assert bf16_round(np.array([2.0 ** -133]))[0] == 2.0 ** -133       # smallest BF16 subnormal
