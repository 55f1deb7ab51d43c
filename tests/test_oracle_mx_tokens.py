"""Pins for the oracle's token-orientation MXFP8 quantizer (the P V operand's V: one E8M0 scale
per 32 consecutive tokens of a sequence, per head and head_dim column).

LP-FA4 README, section "MXFP8 forward and backward": V goes through the same
quantizer as Q and K, and every tensor keeps both hardware orientations. The
token orientation is pinned against the head_dim orientation (itself pinned by
hand-computed blocks) through a transposition: quantizing a (tokens x 128) slice
along tokens is the head_dim quantizer applied to its transpose. Also hand cases,
the padded scale layout, per-sequence independence, and the mx-mode attention
reducing exactly to the fp8 mode when every block scale is 1.
"""
import numpy as np
import pytest

from oracle import (attention_varlen, e4m3_cast, e4m3_decode, mx_dequantize_varlen_tokens,
                    mx_quantize_varlen, mx_quantize_varlen_tokens, scale_offsets)
from synth import bf16_bits_to_f32, make_custom


@pytest.mark.parametrize("mode", ["rceil", "floor"])
@pytest.mark.parametrize("length", [32, 96, 45, 7])
def test_transpose_identity(mode, length):
    """Token blocks of a slice == head_dim blocks of its transpose (zero rows pad the transpose to
    whole blocks; zeros change neither a block maximum nor the real elements' codes)."""
    wl = make_custom([length], [length], heads=2, seed=20 + length)
    x = bf16_bits_to_f32(wl.q_bits).astype(np.float64)           # (L, 2, 128)
    payload, scales, _ = mx_quantize_varlen_tokens(x, np.array([0, length]), mode)
    lp = -(-length // 32) * 32
    for h in range(2):
        xt = np.zeros((128, 1, lp))
        xt[:, 0, :length] = x[:, h, :].T                           # (d, 1, tokens)
        pt, st, _ = mx_quantize_varlen(xt, np.array([0, 128]), mode)
        assert np.array_equal(pt[:, 0, :length].T, payload[:, h, :])
        # head_dim-orientation scale (row d, block b) == token-orientation scale (block b, column d)
        assert np.array_equal(st[:128, 0, :].T, scales[:lp // 32, h, :])


def test_hand_cases():
    """Column 0: a 32-token block with maximum 448 (e = 0, codes exact) then a 3-token block with
    maximum 1.0 (RCEIL: 1 <= 448 * 2^-8, 1 > 448 * 2^-9, so e = -8, byte 0x77; 1.0 * 2^8 = 256 is
    code 0x78; 0.75 * 256 = 192 = 1.5 * 2^7 has exponent field 14 and mantissa 4, code 0x74, so -192
    is 0xF4). Column 1 is all zero: e = -127, byte 0x00, code 0."""
    x = np.zeros((35, 1, 128))
    x[:32, 0, 0] = np.linspace(-448.0, 448.0, 32).round()          # integers up to 448
    x[5, 0, 0] = 448.0
    x[32:, 0, 0] = [1.0, -0.75, 0.5]
    payload, scales, cu_scale = mx_quantize_varlen_tokens(x, np.array([0, 35]), "rceil")
    assert list(cu_scale) == [0, 128]
    assert scales.shape == (4, 1, 128)
    assert scales[0, 0, 0] == 0x7F and scales[1, 0, 0] == 0x77
    assert np.all(scales[0:2, 0, 1] == 0x00) and np.all(payload[:, 0, 1] == 0)
    assert np.all(scales[2:, 0, :] == 0x7F)                        # rows past the last block
    assert payload[5, 0, 0] == 0x7E                                 # 448
    assert list(payload[32:, 0, 0]) == [0x78, 0xF4, 0x70]          # 256, -192, 128
    deq = mx_dequantize_varlen_tokens(payload, scales, np.array([0, 35]))
    assert np.allclose(deq[32:, 0, 0], [1.0, -0.75, 0.5], rtol=0, atol=0)


def test_layout_padding_and_sequence_independence():
    lengths = [5, 128, 129, 0, 300]
    wl = make_custom(lengths, lengths, heads=2, seed=21)
    x = bf16_bits_to_f32(wl.q_bits).astype(np.float64)
    cu = wl.cu_q
    payload, scales, cu_scale = mx_quantize_varlen_tokens(x, cu, "rceil")
    assert np.array_equal(cu_scale, scale_offsets(lengths))
    assert scales.shape == (int(cu_scale[-1]) // 32, 2, 128)
    for i, length in enumerate(lengths):
        r0, r1 = int(cu_scale[i]) // 32, int(cu_scale[i + 1]) // 32
        nblk = -(-length // 32)
        assert np.all(scales[r0 + nblk:r1] == 0x7F)
        c0 = int(cu[i])
        pi, si, _ = mx_quantize_varlen_tokens(x[c0:c0 + length], np.array([0, length]), "rceil")
        assert np.array_equal(pi, payload[c0:c0 + length])
        assert np.array_equal(si[:nblk], scales[r0:r0 + nblk])


def test_last_block_ignores_the_next_sequence():
    """A sequence's last, partial 32-token block takes its maximum over its own tokens only: the
    next sequence (here 2^10 times larger) changes neither its scales nor its codes."""
    lengths = [45, 40]
    wl = make_custom(lengths, lengths, heads=2, seed=22)
    x = bf16_bits_to_f32(wl.q_bits).astype(np.float64)
    x[45:] *= 2.0 ** 10
    payload, scales, _ = mx_quantize_varlen_tokens(x, np.array([0, 45, 85]), "rceil")
    p0, s0, _ = mx_quantize_varlen_tokens(x[:45], np.array([0, 45]), "rceil")
    assert np.array_equal(scales[:2], s0[:2]) and np.array_equal(payload[:45], p0)


@pytest.mark.parametrize("mode", ["rceil", "floor"])
def test_dequant_error_bound(mode):
    """A round-to-nearest E4M3 code is within half its spacing; below the block maximum that is at most
    2^-4 of the value's power-of-two range, plus the saturation error (FLOOR only) above 448 * 2^e."""
    wl = make_custom([77], [77], heads=2, seed=22)
    x = bf16_bits_to_f32(wl.q_bits).astype(np.float64) * 3.0
    p, s, _ = mx_quantize_varlen_tokens(x, np.array([0, 77]), mode)
    deq = mx_dequantize_varlen_tokens(p, s, np.array([0, 77]))
    e = s.astype(np.int64) - 127                                      # (blocks, H, D)
    ee = np.repeat(e, 32, axis=0)[:77]
    step = np.maximum(np.exp2(np.floor(np.log2(np.maximum(np.abs(x) * np.exp2(-ee), 2.0 ** -6))) - 3), 2.0 ** -9)
    bound = 0.5 * step * np.exp2(ee)
    over = np.maximum(np.abs(x) - 448.0 * np.exp2(ee), 0.0)             # FLOOR saturation
    assert np.all(np.abs(deq - x) <= bound + over + 1e-300)
    if mode == "rceil":
        assert np.all(over == 0.0)


def test_mx_mode_equals_fp8_mode_at_unit_scales():
    """V whose every 32-token column block has its maximum in (224, 448] and E4M3 values: RCEIL gives
    e = 0, the payload is the plain E4M3 cast, and the mx-mode attention equals the fp8 mode."""
    rng = np.random.default_rng(23)
    lq, lk, h = 40, 70, 2
    codes = rng.integers(0, 0x7E, size=(lk, h, 128))
    v = e4m3_decode(codes.astype(np.uint8)) * np.where(rng.random((lk, h, 128)) < 0.5, -1.0, 1.0)
    for b in range(0, lk, 32):
        v[b, :, :] = 448.0                                            # block maxima exactly 448
    q = rng.standard_normal((lq, h, 128)) * 0.1
    k = rng.standard_normal((lk, h, 128)) * 0.1
    cu_q, cu_k = np.array([0, lq]), np.array([0, lk])
    p, s, _ = mx_quantize_varlen_tokens(v, cu_k, "rceil")
    assert np.all(s[:3] == 0x7F)
    assert np.array_equal(p, e4m3_cast(v))
    vm = mx_dequantize_varlen_tokens(p, s, cu_k)
    a = attention_varlen(q, k, vm, cu_q, cu_k, pv_mode="mx")
    b = attention_varlen(q, k, e4m3_decode(e4m3_cast(v)), cu_q, cu_k, pv_mode="fp8")
    assert np.array_equal(a.out, b.out) and np.array_equal(a.lse, b.lse)
