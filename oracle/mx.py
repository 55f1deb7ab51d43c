"""MXFP8 block quantization of packed variable-length tensors, float64 — test infrastructure only.

LP-FA4 README, section "MXFP8 forward and backward": inputs are packed
(tokens, heads, 128) BF16 or FP32 tensors; the payload is E4M3 with one E8M0
scale per 32-element block (along head_dim); every sequence gets its own scale
storage padded to a multiple of 128 tokens; RCEIL scale selection is the
default and FLOOR is optional.

Readings (the page names RCEIL and FLOOR without defining them):
* RCEIL: the block exponent e is the smallest integer with amax <= 448 * 2^e, so
  the largest element of a block never saturates (448 * 2^k gives e = k).
* FLOOR (OCP MX v1.0 rule): e = floor(log2(amax)) - 8, so the largest element
  lands in [256, 512) and saturates to 448 when above it.
* e is clamped to [-127, 127]; an all-zero block (amax = 0) gets e = -127.
* scale byte = e + 127; payload = E4M3(x * 2^-e) (x * 2^-e is exact, so there is a
  single rounding).
* Scale layout: (sum_i P(L_i), heads, 4) bytes, P(L) = ceil(L/128)*128; token t of
  sequence i sits at row cu_scale[i] + (t - cu_seqlens[i]); pad rows hold 0x7F.
"""
from __future__ import annotations

from typing import Optional, Tuple

import numpy as np

from .fp8 import E4M3_MAX, e4m3_encode, e4m3_decode, e8m0_decode

BLOCK = 32
PAD = 128
PAD_SCALE_BYTE = 0x7F


def padded_len(length: int) -> int:
    """P(L): length rounded up to a multiple of 128 tokens."""
    return -(-int(length) // PAD) * PAD


def scale_offsets(lengths) -> np.ndarray:
    """cu_scale: prefix sums of P(L_i), int64 of size n+1."""
    out = np.zeros(len(lengths) + 1, dtype=np.int64)
    out[1:] = np.cumsum([padded_len(v) for v in lengths])
    return out


def mx_block_exponent(amax: np.ndarray, mode: str = "rceil") -> np.ndarray:
    """Shared block exponent e (int64) for block maxima ``amax`` >= 0 (float64)."""
    amax = np.asarray(amax, dtype=np.float64)
    e = np.full(amax.shape, -127, dtype=np.int64)
    nz = amax > 0
    a = amax[nz]
    if mode == "rceil":
        # start from a float estimate, then settle with exact comparisons against 448 * 2^e
        est = np.ceil(np.log2(a) - np.log2(E4M3_MAX)).astype(np.int64)
        for _ in range(3):
            too_small = a > np.ldexp(E4M3_MAX, est)              # need a larger e
            est = np.where(too_small, est + 1, est)
            can_lower = a <= np.ldexp(E4M3_MAX, est - 1)         # a smaller e still fits
            est = np.where(can_lower, est - 1, est)
        assert np.all(a <= np.ldexp(E4M3_MAX, est)) and np.all(a > np.ldexp(E4M3_MAX, est - 1))
        e[nz] = est
    elif mode == "floor":
        _, ex = np.frexp(a)                                       # a = f * 2^ex, 0.5 <= f < 1
        e[nz] = (ex - 1) - 8                                      # floor(log2 a) - 8
    else:
        raise ValueError(f"unknown scaling mode {mode!r}")
    return np.clip(e, -127, 127)


def mx_quantize_varlen(x: np.ndarray, cu_seqlens: np.ndarray, mode: str = "rceil"
                       ) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Quantize packed x (T, H, 128) to (payload uint8 (T,H,128), scales uint8 (S,H,4), cu_scale).

    ``x`` holds the exact input values (BF16 or FP32 widened to float64).
    """
    x = np.asarray(x, dtype=np.float64)
    if x.ndim != 3 or x.shape[2] % BLOCK:
        raise ValueError("x must be (tokens, heads, multiple of 32)")
    if not np.all(np.isfinite(x)):
        raise ValueError("non-finite input is outside the method's domain")
    t, h, d = x.shape
    nb = d // BLOCK
    lengths = np.diff(np.asarray(cu_seqlens, dtype=np.int64))
    if cu_seqlens[0] != 0 or cu_seqlens[-1] != t or np.any(lengths < 0):
        raise ValueError("cu_seqlens must run from 0 to tokens, non-decreasing")
    blocks = x.reshape(t, h, nb, BLOCK)
    amax = np.abs(blocks).max(axis=3)                            # (T, H, nb)
    e = mx_block_exponent(amax, mode)
    scaled = blocks * np.ldexp(1.0, -e)[..., None]               # exact: power-of-two scaling
    payload = e4m3_encode(scaled).reshape(t, h, d)
    cu_scale = scale_offsets(lengths)
    scales = np.full((int(cu_scale[-1]), h, nb), PAD_SCALE_BYTE, dtype=np.uint8)
    for i, length in enumerate(lengths):
        s0, c0 = int(cu_scale[i]), int(cu_seqlens[i])
        scales[s0:s0 + length] = (e[c0:c0 + length] + 127).astype(np.uint8)
    return payload, scales, cu_scale


def mx_dequantize_varlen(payload: np.ndarray, scales: np.ndarray, cu_seqlens: np.ndarray,
                         cu_scale: Optional[np.ndarray] = None) -> np.ndarray:
    """payload * 2^(scale - 127) per block, float64 (T, H, 128)."""
    t, h, d = payload.shape
    nb = d // BLOCK
    lengths = np.diff(np.asarray(cu_seqlens, dtype=np.int64))
    if cu_scale is None:
        cu_scale = scale_offsets(lengths)
    vals = e4m3_decode(payload).reshape(t, h, nb, BLOCK)
    out = np.empty_like(vals)
    for i, length in enumerate(lengths):
        s0, c0 = int(cu_scale[i]), int(cu_seqlens[i])
        mult = e8m0_decode(scales[s0:s0 + length])               # (L, H, nb)
        out[c0:c0 + length] = vals[c0:c0 + length] * mult[..., None]
    return out.reshape(t, h, d)


def mx_quantize_varlen_tokens(x: np.ndarray, cu_seqlens: np.ndarray, mode: str = "rceil"
                              ) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Token-orientation MXFP8 of packed x (T, H, 128): one E8M0 scale per 32 consecutive tokens
    of a sequence, per (head, d) — the orientation whose blocks run along the P V contraction.

    LP-FA4 README, section "MXFP8 forward and backward": V is quantized by the same
    routine as Q and K, and each tensor keeps both hardware orientations that the
    forward and backward passes use. The P V product contracts over tokens, so its
    V operand takes blocks of 32 along tokens.

    Readings (the page gives no layout for this orientation):
    * blocks start at each sequence's first token; the last block of a sequence may hold
      fewer than 32 real tokens, and its maximum covers those only;
    * exponent, scale byte and payload follow the same rules as the head_dim orientation
      (``mx_block_exponent``; payload = E4M3(x * 2^-e), one rounding);
    * scale layout: (sum_i P(L_i) / 32, H, 128) bytes; block b of sequence i sits at row
      cu_scale[i] / 32 + b (cu_scale: prefix sums of P(L_i)); rows past a sequence's last
      block hold 0x7F;
    * the payload (T, H, 128) is packed like the input (no padding).
    Returns (payload, scales, cu_scale).
    """
    x = np.asarray(x, dtype=np.float64)
    if x.ndim != 3:
        raise ValueError("x must be (tokens, heads, head_dim)")
    if not np.all(np.isfinite(x)):
        raise ValueError("non-finite input is outside the method's domain")
    t, h, d = x.shape
    lengths = np.diff(np.asarray(cu_seqlens, dtype=np.int64))
    if cu_seqlens[0] != 0 or cu_seqlens[-1] != t or np.any(lengths < 0):
        raise ValueError("cu_seqlens must run from 0 to tokens, non-decreasing")
    cu_scale = scale_offsets(lengths)
    payload = np.zeros((t, h, d), dtype=np.uint8)
    scales = np.full((int(cu_scale[-1]) // BLOCK, h, d), PAD_SCALE_BYTE, dtype=np.uint8)
    for i, length in enumerate(lengths):
        c0, row0 = int(cu_seqlens[i]), int(cu_scale[i]) // BLOCK
        for b in range(-(-int(length) // BLOCK)):
            lo, hi = c0 + BLOCK * b, c0 + min(BLOCK * (b + 1), int(length))
            block = x[lo:hi]                                      # (<= 32 tokens, H, D)
            e = mx_block_exponent(np.abs(block).max(axis=0), mode)   # (H, D)
            payload[lo:hi] = e4m3_encode(block * np.ldexp(1.0, -e)[None])
            scales[row0 + b] = (e + 127).astype(np.uint8)
    return payload, scales, cu_scale


def mx_dequantize_varlen_tokens(payload: np.ndarray, scales: np.ndarray, cu_seqlens: np.ndarray,
                                cu_scale: Optional[np.ndarray] = None) -> np.ndarray:
    """payload * 2^(scale - 127) with the scale of each token's 32-token block, float64 (T, H, 128)."""
    t, h, d = payload.shape
    lengths = np.diff(np.asarray(cu_seqlens, dtype=np.int64))
    if cu_scale is None:
        cu_scale = scale_offsets(lengths)
    vals = e4m3_decode(payload)
    out = np.empty_like(vals)
    for i, length in enumerate(lengths):
        c0, row0 = int(cu_seqlens[i]), int(cu_scale[i]) // BLOCK
        for j in range(int(length)):
            out[c0 + j] = vals[c0 + j] * e8m0_decode(scales[row0 + j // BLOCK])
    return out


def e4m3_cast(x: np.ndarray) -> np.ndarray:
    """Unscaled cast to E4M3 codes (the fp8 PV mode's V): round to nearest even, saturate at 448.

    FastVideo fp8-PV PR: the V cast carries no scale factors; the kernel reads it
    with an implicit dequant scale of 1.0.
    """
    return e4m3_encode(np.asarray(x, dtype=np.float64))


def pertensor_quantize(x: np.ndarray, cu_seqlens: np.ndarray, descale: Optional[np.ndarray]
                       ) -> np.ndarray:
    """Per-(sequence, head) FP8 input preparation: E4M3(x / s) with s = descale[seq, head] (1 if None).

    This prepares the per-tensor workload's inputs (the vLLM descale PR passes
    q/k/v descales of shape (num_seqs, num_kv_heads)); dequantizing multiplies
    by the same s.
    """
    x = np.asarray(x, dtype=np.float64)
    if descale is None:
        return e4m3_encode(x)
    lengths = np.diff(np.asarray(cu_seqlens, dtype=np.int64))
    per_token = np.repeat(np.asarray(descale, dtype=np.float64), lengths, axis=0)   # (T, H)
    return e4m3_encode(x / per_token[..., None])
