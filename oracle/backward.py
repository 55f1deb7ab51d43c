"""Noncausal varlen attention backward on dequantized MXFP8 operands, float64 — test infrastructure only.

What is computed (LP-FA4 README, section "MXFP8 forward and backward"): the backward takes the
quantized Q, K and V, each kept in the two hardware orientations that the forward and backward
products need, together with the forward's BF16 output, the output gradient and the LSE. It
returns dQ in BF16, and dK and dV either in BF16 or as E4M3 payloads with one E8M0 scale per
32-element block (the ``output_mxfp8_dkv`` option). The gradients are those of the forward
O = softmax(tau Q K^T) V, written as the usual recomputation from the saved LSE:

    s_ij  = tau * (Qd_i . Kd_j)             scores from the head_dim orientation, as in the forward
    P_ij  = exp(s_ij - LSE_i)               the forward's LSE (natural log)
    dP_ij = dO_i . Vd_j                     V's head_dim orientation (the contraction runs over d)
    D_i   = dO_i . O_i                      the forward's output as given
    dS_ij = P_ij * (dP_ij - D_i)
    dV_j  = sum_i r(P_ij) dO_i
    dK_j  = tau * sum_i r(dS_ij) Qt_i       Q's token orientation (the contraction runs over queries)
    dQ_i  = tau * sum_j r(dS_ij) Kt_j       K's token orientation (the contraction runs over keys)

r() is the rounding of the probabilities and score gradients to the matrix operand type:
BF16 (nearest even) by default, as the forward's bf16 P V mode rounds P; ``round_ops="none"``
keeps them exact (used to pin the formulas against the derivative of the forward).

Readings (the page gives the API and the output formats, not the arithmetic):
* the token orientation is the one whose 32-element blocks run along the contraction of the
  product it feeds (dK contracts over queries, dQ over keys), the head_dim orientation serves
  the products that contract over head_dim (S and dP), as in the forward;
* dO is used as given (BF16), unquantized; D uses the given output, not a recomputed one;
* queries of sequence r attend to the keys of sequence r only; the query and key lengths may
  differ; a sequence with queries but no keys is rejected, one with keys but no queries gets
  zero dK and dV;
* tau defaults to 1/sqrt(head_dim).
All operands are passed in as float64 (the dequantized values; dO, O and LSE as stored).
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional, Sequence

import numpy as np

from .fp8 import bf16_round


@dataclass
class BackwardResult:
    dq: np.ndarray   # (Tq, H, D) float64
    dk: np.ndarray   # (Tk, H, D) float64
    dv: np.ndarray   # (Tk, H, D) float64


def _round_ops(x: np.ndarray, mode: str) -> np.ndarray:
    if mode == "bf16":
        return bf16_round(x)
    if mode == "none":
        return x
    raise ValueError(f"unknown round_ops {mode!r}")


def attention_varlen_bwd(qd: np.ndarray, kd: np.ndarray, vd: np.ndarray,
                         qt: np.ndarray, kt: np.ndarray,
                         out: np.ndarray, dout: np.ndarray, lse: np.ndarray,
                         cu_q: Sequence[int], cu_k: Sequence[int],
                         softmax_scale: Optional[float] = None,
                         round_ops: str = "bf16") -> BackwardResult:
    """Gradients of the packed-sequence attention forward.

    qd, kd, vd: head_dim-orientation operands (Tq|Tk, H, D); qt, kt: token-orientation Q and K;
    out, dout: (Tq, H, D); lse: (H, Tq) natural-log LSE of the scaled scores.
    """
    f = lambda a: np.asarray(a, dtype=np.float64)
    qd, kd, vd, qt, kt, out, dout, lse = map(f, (qd, kd, vd, qt, kt, out, dout, lse))
    tq, h, d = qd.shape
    tk = kd.shape[0]
    tau = 1.0 / np.sqrt(d) if softmax_scale is None else float(softmax_scale)
    cu_q = np.asarray(cu_q, dtype=np.int64)
    cu_k = np.asarray(cu_k, dtype=np.int64)
    dq = np.zeros((tq, h, d))
    dk = np.zeros((tk, h, d))
    dv = np.zeros((tk, h, d))
    for r in range(len(cu_q) - 1):
        q0, q1 = int(cu_q[r]), int(cu_q[r + 1])
        k0, k1 = int(cu_k[r]), int(cu_k[r + 1])
        if q1 == q0:
            continue
        if k1 == k0:
            raise ValueError(f"sequence {r} has queries but no keys")
        for hh in range(h):
            Qd, Kd, Vd = qd[q0:q1, hh], kd[k0:k1, hh], vd[k0:k1, hh]
            Qt, Kt = qt[q0:q1, hh], kt[k0:k1, hh]
            O, dO = out[q0:q1, hh], dout[q0:q1, hh]
            s = tau * (Qd @ Kd.T)
            p = np.exp(s - lse[hh, q0:q1][:, None])
            dp = dO @ Vd.T
            D = np.sum(dO * O, axis=1)
            ds = p * (dp - D[:, None])
            pr, dsr = _round_ops(p, round_ops), _round_ops(ds, round_ops)
            dv[k0:k1, hh] = pr.T @ dO
            dk[k0:k1, hh] = tau * (dsr.T @ Qt)
            dq[q0:q1, hh] = tau * (dsr @ Kt)
    return BackwardResult(dq, dk, dv)
