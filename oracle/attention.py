"""Noncausal varlen attention forward with PV-mode probability rounding, float64 — test infrastructure only.

What is computed (LP-FA4 README, introduction and section "MXFP8 forward and
backward": noncausal head_dim-128 MHA over packed sequences, returning (out,
lse); FastVideo fp8-PV PR: V is BF16 in the default mode or an unscaled E4M3
cast in the fp8 mode, and the output is BF16 either way; vLLM unit-descale PR:
optional per-tensor q/k/v descales, a missing one reading as 1.0):

    s_ij  = softmax_scale * qd * kd * (Qhat_i . Khat_j)
    m_i   = max_j s_ij                      (the final row maximum: plain two-pass softmax)
    u_ij  = exp(s_ij - m_i)
    l_i   = sum_j u_ij                      (unrounded)
    P_ij  = round_pv(u_ij)                  (BF16 in the bf16 mode, E4M3 unscaled in the fp8 and mx modes)
    O_i   = vd * (sum_j P_ij V'_j) / l_i
    LSE_i = m_i + ln(l_i)                   (natural log of the sum of exp of the scaled scores)

Readings: softmax_scale defaults to 1/sqrt(head_dim); the probabilities take
V's matrix-multiply type; LSE is laid out (heads, query tokens); queries of
sequence r attend to the keys of sequence r only, and the query and key
lengths may differ. A sequence with queries but no keys has no defined output
and is rejected.

Qhat/Khat are the dequantized operands (MX payload times block scale, or the
per-tensor payload), V' is the BF16 V (bf16 mode), its E4M3 cast (fp8 mode) or
its dequantized token-orientation MXFP8 (mx mode: the LP-FA4 forward's v_mx
operand, one scale per 32 tokens), all passed in as float64.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Dict, Optional, Sequence

import numpy as np

from .fp8 import bf16_round, e4m3_encode, e4m3_decode


@dataclass
class AttentionResult:
    out: np.ndarray        # (Tq, H, D) float64, NaN for query rows not computed
    lse: np.ndarray        # (H, Tq) float64, NaN for rows not computed


def _round_pv(u: np.ndarray, pv_mode: str) -> np.ndarray:
    if pv_mode == "bf16":
        return bf16_round(u)
    if pv_mode in ("fp8", "mx"):
        # mx: V MXFP8 along tokens; the probabilities stay unscaled E4M3 as in the fp8 mode
        return e4m3_decode(e4m3_encode(u))
    raise ValueError(f"unknown pv_mode {pv_mode!r}")


def _descale(d: Optional[np.ndarray], r: int, h: int) -> float:
    return 1.0 if d is None else float(np.asarray(d, dtype=np.float64)[r, h])


def attention_varlen(qhat: np.ndarray, khat: np.ndarray, vprime: np.ndarray,
                     cu_q: Sequence[int], cu_k: Sequence[int], pv_mode: str = "bf16",
                     softmax_scale: Optional[float] = None,
                     q_descale: Optional[np.ndarray] = None,
                     k_descale: Optional[np.ndarray] = None,
                     v_descale: Optional[np.ndarray] = None,
                     rows: Optional[Dict[int, np.ndarray]] = None,
                     row_block: int = 1024) -> AttentionResult:
    """Attention over packed sequences.

    ``rows`` optionally restricts the computation to given local query indices per
    sequence ({seq: indices}); rows not listed stay NaN. ``row_block`` bounds the
    score matrix held at once (rows are independent; only float64 rounding of the
    library matmul can differ with the block shape).
    Descales have shape (num_seqs, heads).
    """
    qhat = np.asarray(qhat, dtype=np.float64)
    khat = np.asarray(khat, dtype=np.float64)
    vprime = np.asarray(vprime, dtype=np.float64)
    tq, h, d = qhat.shape
    if softmax_scale is None:
        softmax_scale = 1.0 / np.sqrt(d)
    cu_q = np.asarray(cu_q, dtype=np.int64)
    cu_k = np.asarray(cu_k, dtype=np.int64)
    out = np.full((tq, h, d), np.nan)
    lse = np.full((h, tq), np.nan)
    for r in range(len(cu_q) - 1):
        q0, q1 = int(cu_q[r]), int(cu_q[r + 1])
        k0, k1 = int(cu_k[r]), int(cu_k[r + 1])
        if q1 == q0:
            continue
        if k1 == k0:
            raise ValueError(f"sequence {r} has queries but no keys")
        idx = np.arange(q1 - q0) if rows is None else np.asarray(rows.get(r, []), dtype=np.int64)
        for hh in range(h):
            c = softmax_scale * _descale(q_descale, r, hh) * _descale(k_descale, r, hh)
            vd = _descale(v_descale, r, hh)
            K = khat[k0:k1, hh]
            V = vprime[k0:k1, hh]
            for b0 in range(0, len(idx), row_block):
                sel = idx[b0:b0 + row_block]
                Q = qhat[q0 + sel, hh]
                s = c * (Q @ K.T)
                m = s.max(axis=1)
                u = np.exp(s - m[:, None])
                l = u.sum(axis=1)
                p = _round_pv(u, pv_mode)
                out[q0 + sel, hh] = vd * (p @ V) / l[:, None]
                lse[hh, q0 + sel] = m + np.log(l)
    return AttentionResult(out, lse)
