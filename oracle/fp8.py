"""Number formats of the path: E4M3 (OCP E4M3FN), E8M0 and BF16, in float64.

Test infrastructure only (see the package docstring).

The LP-FA4 README (section "MXFP8 forward and backward") names the formats: E4M3
payloads and E8M0 block scales. The FastVideo fp8-PV PR casts V with
``.to(torch.float8_e4m3fn)``, i.e. the OCP "FN" variant: no infinities, a single
NaN pattern per sign (0x7F / 0xFF), largest finite magnitude 448.

Readings (the pages name the formats but not their rounding):
* Encoding rounds to the nearest representable value, ties to the code with an
  even mantissa (even code), and saturates finite magnitudes above 448 to 448.
  The sign is kept, so negative values that round to zero give 0x80.
* E8M0 byte b encodes 2^(b-127) for b in 0..254 (0xFF is NaN and never produced).
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0


def _e4m3_table() -> np.ndarray:
    """Value of every code 0..255 from the field definition (sign, 4-bit exponent bias 7, 3-bit mantissa)."""
    vals = np.empty(256, dtype=np.float64)
    for c in range(256):
        s = -1.0 if c & 0x80 else 1.0
        e = (c >> 3) & 0xF
        m = c & 0x7
        if (c & 0x7F) == 0x7F:
            vals[c] = np.nan
        elif e == 0:
            vals[c] = s * m * 2.0 ** -9          # subnormal: m/8 * 2^(1-7)
        else:
            vals[c] = s * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return vals


E4M3_VALUES = _e4m3_table()
# non-negative finite magnitudes, codes 0x00..0x7E, strictly increasing with the code
_POS = E4M3_VALUES[:0x7F].copy()


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    """E4M3 byte codes -> float64 values (NaN for 0x7F/0xFF)."""
    return E4M3_VALUES[np.asarray(codes, dtype=np.uint8)]


def e4m3_encode(x: np.ndarray) -> np.ndarray:
    """Float64 -> E4M3 code: nearest finite code, ties to even code, saturating at 448, sign kept.

    The nearest code is found by locating |x| between the two neighbouring table
    magnitudes. Input must be finite.
    """
    x = np.asarray(x, dtype=np.float64)
    if not np.all(np.isfinite(x)):
        raise ValueError("e4m3_encode: non-finite input")
    a = np.abs(x)
    hi = np.searchsorted(_POS, a, side="left")          # first magnitude >= a
    hi = np.minimum(hi, 0x7E)
    lo = np.maximum(hi - 1, 0)
    d_hi = _POS[hi] - a
    d_lo = a - _POS[lo]
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo)
    code = np.where(a >= E4M3_MAX, 0x7E, code)           # saturation (448 itself is code 0x7E)
    code = np.where(np.signbit(x), code | 0x80, code)
    return code.astype(np.uint8)


def e8m0_decode(b: np.ndarray) -> np.ndarray:
    """E8M0 byte -> 2^(b-127) in float64."""
    b = np.asarray(b, dtype=np.int64)
    if np.any(b == 255):
        raise ValueError("e8m0_decode: NaN scale byte")
    return np.ldexp(1.0, b - 127)


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round float64 values to the nearest BF16 value (ties to even), returned as float64.

    BF16 keeps 8 significant bits and float32's exponent range; below 2^-126 the
    spacing is that of its subnormals, 2^-133. Used for the probabilities in the
    bf16 PV mode. Values must be finite and below the BF16 overflow threshold.
    """
    x = np.asarray(x, dtype=np.float64)
    _, e = np.frexp(x)                                   # x = f * 2^e, 0.5 <= |f| < 1
    quantum = np.ldexp(1.0, np.maximum(e - 8, -133))
    return np.rint(x / quantum) * quantum                # rint: half to even


def bf16_encode(x: np.ndarray) -> np.ndarray:
    """Float64 -> BF16 bit patterns (uint16) via :func:`bf16_round` (exact once rounded)."""
    r = bf16_round(x).astype(np.float32)
    return (r.view(np.uint32) >> 16).astype(np.uint16)
