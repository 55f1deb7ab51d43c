"""Shared test helpers: upload synthetic workloads, run the oracle on them, compare within tolerance."""
from __future__ import annotations

import json
import os
from typing import Dict, Optional

import numpy as np
import torch

import oracle
from synth import Workload, bf16_bits_to_f32

# Tolerances of the attention output against the oracle (absolute): O max 2e-2, O mean 2e-3,
# LSE max 1e-3.
O_MAX_ABS = 2e-2
O_MEAN_ABS = 2e-3
LSE_MAX_ABS = 1e-3


def bf16_to_device(bits: np.ndarray, dev="cuda") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16).copy()).view(torch.bfloat16).to(dev)


def f64(bits: np.ndarray) -> np.ndarray:
    return bf16_bits_to_f32(bits).astype(np.float64)


def oracle_operands(wl: Workload, pv_mode: str, mode: str = "mx", descales: Optional[Dict] = None):
    """Oracle Qhat, Khat, V' (float64) and the bytes the GPU path should produce or consume."""
    xq, xk, xv = f64(wl.q_bits), f64(wl.k_bits), f64(wl.v_bits)
    res = {}
    if mode == "mx":
        pq, sq, csq = oracle.mx_quantize_varlen(xq, wl.cu_q)
        pk, sk, csk = oracle.mx_quantize_varlen(xk, wl.cu_k)
        res.update(pq=pq, sq=sq, pk=pk, sk=sk)
        res["qhat"] = oracle.mx_dequantize_varlen(pq, sq, wl.cu_q, csq)
        res["khat"] = oracle.mx_dequantize_varlen(pk, sk, wl.cu_k, csk)
    else:
        d = descales or {"q": None, "k": None, "v": None}
        pq = oracle.pertensor_quantize(xq, wl.cu_q, d["q"])
        pk = oracle.pertensor_quantize(xk, wl.cu_k, d["k"])
        res.update(pq=pq, pk=pk)
        res["qhat"] = oracle.e4m3_decode(pq)
        res["khat"] = oracle.e4m3_decode(pk)
    if pv_mode == "mx":   # V MXFP8 along tokens (the oracle's token orientation)
        pv, sv, csv = oracle.mx_quantize_varlen_tokens(xv, wl.cu_k)
        res.update(pv=pv, sv=sv)
        res["vprime"] = oracle.mx_dequantize_varlen_tokens(pv, sv, wl.cu_k, csv)
    elif pv_mode == "fp8":
        if mode == "mx":
            pv = oracle.e4m3_cast(xv)
        else:
            d = descales or {"v": None}
            pv = oracle.pertensor_quantize(xv, wl.cu_k, d["v"])
        res["pv"] = pv
        res["vprime"] = oracle.e4m3_decode(pv)
    else:
        res["vprime"] = xv
    return res


def bf16_ulp(x: np.ndarray) -> np.ndarray:
    """The BF16 spacing at |x| (8 significant bits)."""
    _, e = np.frexp(np.abs(x))
    return np.ldexp(1.0, np.maximum(e - 8, -133))


def compare(out: torch.Tensor, lse: torch.Tensor, ref: oracle.AttentionResult, rows=None, cu_q=None):
    """Max/mean absolute O error and max LSE error over the rows the oracle computed.

    Also reports o_max_beyond_bf16: the largest O error after subtracting one BF16 ulp of the
    oracle value (the output's own rounding plus as much again for the BF16-rounded probabilities
    it was accumulated from), and how many elements exceed the plain absolute bound."""
    o = out.float().cpu().numpy().astype(np.float64)
    l = lse.cpu().numpy().astype(np.float64)
    mask = ~np.isnan(ref.lse[0])
    do = np.abs(o[mask] - ref.out[mask])
    dl = np.abs(l[:, mask] - ref.lse[:, mask])
    allow = bf16_ulp(ref.out[mask])
    return {"o_max": float(do.max()), "o_mean": float(do.mean()), "lse_max": float(dl.max()),
            "rows": int(mask.sum()), "o_rel": float(np.linalg.norm(o[mask] - ref.out[mask]) /
                                                   max(np.linalg.norm(ref.out[mask]), 1e-300)),
            "o_max_beyond_bf16": float((do - allow).max()),
            "n_over_abs": int((do > O_MAX_ABS).sum()),
            "max_abs_ref": float(np.abs(ref.out[mask]).max())}


def record(stats, name=None):
    """Append parity statistics to $LPFA_PARITY_LOG (one JSON line per comparison), if set."""
    path = os.environ.get("LPFA_PARITY_LOG")
    if path:
        entry = dict(stats)
        entry["test"] = name or os.environ.get("PYTEST_CURRENT_TEST", "?").split(" ")[0]
        with open(path, "a") as f:
            f.write(json.dumps(entry) + "\n")


def assert_within(stats, o_max=O_MAX_ABS, o_mean=O_MEAN_ABS, lse_max=LSE_MAX_ABS, bf16_allowance=False):
    """The tolerances on O and LSE. With bf16_allowance, O elements may exceed o_max by one BF16
    ulp at their magnitude: above |O| ~ 4 a BF16 output's own rounding is comparable to o_max, so
    a fixed absolute bound cannot hold there."""
    record(stats)
    if bf16_allowance:
        assert stats["o_max_beyond_bf16"] <= o_max, stats
    else:
        assert stats["o_max"] <= o_max, stats
    assert stats["o_mean"] <= o_mean, stats
    assert stats["lse_max"] <= lse_max, stats
