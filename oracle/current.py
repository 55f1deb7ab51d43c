"""Per-tensor current scaling to E4M3, float32 scale arithmetic — test infrastructure only.

TensorRT-LLM PR "TE FP8 attention backend for VisualGen" (description, "Inference scaling
fix"): with scales left at 1.0, a small attention output loses precision below E4M3's normal
range, so the backend writes the Q, K, V and O scales from the current tensors before every
call. Current scaling maps each tensor's largest magnitude onto the E4M3 maximum.

Readings (the page names the recipe, not its arithmetic):
* one scale per tensor: s = amax / 448, computed in float32 (round to nearest); the payload is
  E4M3(x / s) with the quotient also rounded to float32 first (the codes are decided in the same
  precision on both sides); the element of largest magnitude therefore encodes to +-448;
* an all-zero tensor takes s = 1 (no scaling);
* s is the tensor's descale: x ~ s * decode(payload). The attention consumes it as the per-tensor
  q/k/v descale; for O it is the output's descale (an FP8 O).
"""
from __future__ import annotations

from typing import Tuple

import numpy as np

from .fp8 import E4M3_MAX, e4m3_encode


def current_scale(x: np.ndarray) -> np.float32:
    """s = fl32(amax / 448) of a float tensor (1 for an all-zero tensor)."""
    x = np.asarray(x)
    if not np.all(np.isfinite(x)):
        raise ValueError("non-finite input is outside the method's domain")
    amax = np.float32(np.abs(x.astype(np.float32)).max()) if x.size else np.float32(0.0)
    if amax == 0:
        return np.float32(1.0)
    return np.float32(amax / np.float32(E4M3_MAX))


def current_quantize(x: np.ndarray) -> Tuple[np.ndarray, np.float32]:
    """(E4M3 codes of fl32(x / s), s) with s = current_scale(x); x holds BF16 or FP32 values."""
    s = current_scale(x)
    q = (np.asarray(x, dtype=np.float32) / s).astype(np.float32)   # float32 division, nearest
    return e4m3_encode(q.astype(np.float64)), s
