"""Seeded synthetic inputs shared by the oracle's tests, the GPU tests and the benchmark.

This module only draws random numbers and lays them out. It holds none of the
method's arithmetic: no FP8 encoding, no scale selection and no attention. The
one rounding it performs is the BF16 rounding of the drawn float32 inputs,
because the workloads are defined as BF16 tensors (the LP-FA4 README, section
"MXFP8 forward and backward", takes packed (tokens, heads, 128) BF16 or FP32
inputs).

Workloads (sizes from the five benchmark configurations of this project):

* ``tiny``    one sequence of 256 tokens, 2 heads.
* ``dense``   one sequence of 2048 tokens, 16 heads (dense attention written as
              uniform packed offsets, LP-FA4 README, introduction).
* ``varlen``  8 sequences, lengths drawn uniformly from the integers 128..4096,
              16 heads, 0.1% of entries scaled by 20 as outliers.
* ``pertensor`` 2 sequences of 16384 tokens, 24 heads, per-tensor FP8 (video-DiT
              like); descale cases none / unit / 2^-3 / per-(sequence, head)
              log-uniform in [2^-4, 2^2].
* ``cross``   queries: one sequence of 4096 tokens; keys/values: one sequence of
              32768 tokens; 16 heads; keys drawn with variance 0.25.

Draw order for every workload (one ``numpy.random.default_rng(seed)``):
lengths (varlen only), then Q, K, V normals (float32), then the outlier masks
of Q, K, V (varlen only), then descales (pertensor only). Outliers are applied
in float32 before the single BF16 rounding.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, List, Optional

import numpy as np

HEAD_DIM = 128


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to BF16 (round to nearest, ties to even) and return the uint16 bit patterns.

    Inputs must be finite (all draws here are).
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen BF16 bit patterns to float32 (exact)."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def cu_from_lengths(lengths: List[int]) -> np.ndarray:
    """Prefix sums [0, L0, L0+L1, ...] as int64 (packed token offsets)."""
    cu = np.zeros(len(lengths) + 1, dtype=np.int64)
    cu[1:] = np.cumsum(np.asarray(lengths, dtype=np.int64))
    return cu


@dataclass
class Workload:
    """One synthetic attention problem. Q/K/V are BF16 bit patterns, shape (tokens, heads, 128)."""

    name: str
    lengths_q: List[int]
    lengths_k: List[int]
    num_heads: int
    q_bits: np.ndarray
    k_bits: np.ndarray
    v_bits: np.ndarray
    # pertensor only: descale arrays of shape (num_seqs, num_heads) per case, keyed by case name
    descales: Dict[str, Dict[str, Optional[np.ndarray]]] = field(default_factory=dict)

    @property
    def cu_q(self) -> np.ndarray:
        return cu_from_lengths(self.lengths_q)

    @property
    def cu_k(self) -> np.ndarray:
        return cu_from_lengths(self.lengths_k)

    def flops(self) -> int:
        """4 * Lq * Lk * H * D summed over sequences (noncausal attention forward)."""
        return int(sum(4 * lq * lk * self.num_heads * HEAD_DIM
                       for lq, lk in zip(self.lengths_q, self.lengths_k)))


def _normals(rng: np.random.Generator, tokens: int, heads: int, std: float = 1.0) -> np.ndarray:
    x = rng.standard_normal((tokens, heads, HEAD_DIM), dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return x


def make_workload(name: str, seed: int = 0, scale_tokens: int = 1) -> Workload:
    """Build a named workload. ``scale_tokens`` > 1 divides every sequence length (for small tests)."""
    rng = np.random.default_rng(seed)
    if name == "tiny":
        lq = lk = [256]
        heads = 2
    elif name == "dense":
        lq = lk = [2048]
        heads = 16
    elif name == "varlen":
        lq = lk = [int(v) for v in rng.integers(128, 4097, size=8)]
        heads = 16
    elif name == "pertensor":
        lq = lk = [16384, 16384]
        heads = 24
    elif name == "cross":
        lq, lk = [4096], [32768]
        heads = 16
    elif name == "batch8":  # the LP-FA4 README's bundled benchmark shape: 8 x 2048 tokens, 16 heads
        lq = lk = [2048] * 8
        heads = 16
    else:
        raise ValueError(f"unknown workload {name!r}")
    if scale_tokens > 1:
        lq = [max(1, v // scale_tokens) for v in lq]
        lk = [max(1, v // scale_tokens) for v in lk]
    tq, tk = int(sum(lq)), int(sum(lk))
    q = _normals(rng, tq, heads)
    k = _normals(rng, tk, heads, std=0.5 if name == "cross" else 1.0)
    v = _normals(rng, tk, heads)
    if name == "varlen":
        for x in (q, k, v):
            mask = rng.random(x.shape) < 0.001
            x[mask] *= np.float32(20.0)
    wl = Workload(name, lq, lk, heads, f32_to_bf16_bits(q), f32_to_bf16_bits(k), f32_to_bf16_bits(v))
    if name == "pertensor":
        n = len(lq)
        per_head = {t: np.exp2(rng.uniform(-4.0, 2.0, size=(n, heads))) for t in ("q", "k", "v")}
        wl.descales = {
            "none": {"q": None, "k": None, "v": None},
            "unit": {t: np.ones((n, heads)) for t in ("q", "k", "v")},
            "calibrated": {t: np.full((n, heads), 2.0 ** -3) for t in ("q", "k", "v")},
            "perhead": per_head,
        }
    return wl


def random_lengths(rng: np.random.Generator, n: int, lo: int, hi: int) -> List[int]:
    """n integer lengths drawn uniformly from lo..hi inclusive."""
    return [int(v) for v in rng.integers(lo, hi + 1, size=n)]


def make_custom(lengths_q: List[int], lengths_k: List[int], heads: int, seed: int = 0,
                k_std: float = 1.0, outlier_rate: float = 0.0) -> Workload:
    """A workload of arbitrary lengths, same draw order as the named ones."""
    rng = np.random.default_rng(seed)
    q = _normals(rng, int(sum(lengths_q)), heads)
    k = _normals(rng, int(sum(lengths_k)), heads, std=k_std)
    v = _normals(rng, int(sum(lengths_k)), heads)
    if outlier_rate > 0:
        for x in (q, k, v):
            mask = rng.random(x.shape) < outlier_rate
            x[mask] *= np.float32(20.0)
    return Workload("custom", list(lengths_q), list(lengths_k), heads,
                    f32_to_bf16_bits(q), f32_to_bf16_bits(k), f32_to_bf16_bits(v))


def make_output_grad(tokens: int, heads: int, seed: int = 0, std: float = 1.0) -> np.ndarray:
    """A seeded output gradient dO: N(0, std^2) rounded to BF16 bit patterns, (tokens, heads, 128)
    (the README's backward example draws it as a standard normal like the output)."""
    rng = np.random.default_rng(seed)
    return f32_to_bf16_bits(_normals(rng, tokens, heads, std))
