"""ctypes loader for liblpfa.so (the C ABI declared in include/lpfa.h).

The library is built in-tree by ``precision_attention_mxfp8_amd.build.build_library``.
Loading fails loudly when it is missing: there is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os
import threading

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "liblpfa.so")

LPFA_OK = 0
LPFA_EIO = -5
LPFA_EINVAL = -22
LPFA_ENOTSUP = -95

DTYPE_BF16 = 0
DTYPE_FP32 = 1
SCALING = {"rceil": 0, "floor": 1}
PV_MODES = {"bf16": 0, "fp8": 1, "mx": 2}
ABI_VERSION = 9

EXPORTS = ("lpfa_abi_version", "lpfa_last_error", "mxfp8_quantize_varlen", "mxfp8_quantize_varlen_tokens",
           "mxfp8_prepare_qkv", "lp_fp8_cast_e4m3", "lp_fp8_cast_current", "lp_fp8_cast_current_noalloc", "lp_attn_varlen_fwd",
           "lp_attn_varlen_bwd")

_p = ctypes.c_void_p
_i32 = ctypes.c_int32
_i64 = ctypes.c_int64


class AttnArgs(ctypes.Structure):
    """Mirror of ``lpfa_attn_args`` (same field order and types)."""

    _fields_ = [
        ("struct_size", _i32),
        ("q", _p), ("k", _p),
        ("q_stride_tok", _i64), ("q_stride_head", _i64),
        ("k_stride_tok", _i64), ("k_stride_head", _i64),
        ("q_scale", _p), ("k_scale", _p),
        ("cu_scale_q", _p), ("cu_scale_k", _p),
        ("v", _p),
        ("v_stride_tok", _i64), ("v_stride_head", _i64),
        ("pv_mode", _i32),
        ("cu_seqlens_q", _p), ("cu_seqlens_k", _p),
        ("num_seqs", _i32), ("max_seqlen_q", _i32), ("max_seqlen_k", _i32),
        ("total_q", _i64), ("total_k", _i64),
        ("num_heads", _i32), ("head_dim", _i32),
        ("softmax_scale", ctypes.c_float),
        ("causal", _i32),
        ("q_descale", _p), ("k_descale", _p), ("v_descale", _p),
        ("q_descale_stride_seq", _i64), ("q_descale_stride_head", _i64),
        ("k_descale_stride_seq", _i64), ("k_descale_stride_head", _i64),
        ("v_descale_stride_seq", _i64), ("v_descale_stride_head", _i64),
        ("out", _p), ("lse", _p),
        ("tile_order", _p), ("num_tiles", _i32),
        ("start_event", _p), ("stop_event", _p),
        ("k_scale_group_max", _p),
        ("v_scale", _p),
        ("qk_bf16", _i32),
        ("fp8_score_guard", ctypes.c_float),
        ("k_deq", ctypes.c_void_p),
    ]


class BwdArgs(ctypes.Structure):
    """Mirror of ``lpfa_bwd_args`` (same field order and types)."""

    _fields_ = [
        ("struct_size", _i32),
        ("q", _p), ("q_scale", _p), ("k", _p), ("k_scale", _p), ("v", _p), ("v_scale", _p),
        ("q_t", _p), ("q_t_scale", _p), ("k_t", _p), ("k_t_scale", _p),
        ("out", _p), ("dout", _p), ("lse", _p),
        ("cu_seqlens_q", _p), ("cu_seqlens_k", _p), ("cu_scale_q", _p), ("cu_scale_k", _p),
        ("num_seqs", _i32), ("num_heads", _i32), ("head_dim", _i32), ("causal", _i32),
        ("total_q", _i64), ("total_k", _i64),
        ("total_scale_rows_q", _i64), ("total_scale_rows_k", _i64),
        ("softmax_scale", ctypes.c_float),
        ("output_mxfp8_dkv", _i32), ("scaling_mode", _i32),
        ("work", _p), ("dq", _p), ("dk", _p), ("dv", _p), ("dk_scale", _p), ("dv_scale", _p),
    ]


def bwd_work_bytes(total_q: int, total_k: int, num_heads: int) -> int:
    """LPFA_BWD_WORK_BYTES: D (float32, rounded up to 256 bytes) + five BF16 (tokens, H, 128) copies."""
    return (num_heads * total_q * 4 + 255) // 256 * 256 + num_heads * 256 * (2 * total_q + 3 * total_k)


_lib = None
_lock = threading.Lock()


class LpfaError(RuntimeError):
    """An entry point returned a negative code; ``code`` holds it."""

    def __init__(self, name: str, code: int, msg: str):
        super().__init__(f"{name} failed with code {code}: {msg}")
        self.code = code


def load() -> ctypes.CDLL:
    """Load liblpfa.so once (raises if it was not built)."""
    global _lib
    if _lib is not None:
        return _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                               "(hipcc --offload-arch=gfx950); there is no fallback path")
        lib = ctypes.CDLL(LIB_PATH)
        lib.lpfa_abi_version.restype = ctypes.c_int
        lib.lpfa_abi_version.argtypes = []
        lib.lpfa_last_error.restype = ctypes.c_char_p
        lib.lpfa_last_error.argtypes = []
        lib.mxfp8_quantize_varlen.restype = ctypes.c_int
        lib.mxfp8_quantize_varlen.argtypes = [_p, ctypes.c_int, _i64, _i64, _i64, _i32, _i32, _p, _p,
                                              _i32, _i64, ctypes.c_int, _p, _p, _p, _p, _p]
        lib.mxfp8_quantize_varlen_tokens.restype = ctypes.c_int
        lib.mxfp8_quantize_varlen_tokens.argtypes = [_p, ctypes.c_int, _i64, _i64, _i64, _i32, _i32, _p, _p,
                                                     _i32, _i64, ctypes.c_int, _p, _p, _p]
        lib.mxfp8_prepare_qkv.restype = ctypes.c_int
        lib.mxfp8_prepare_qkv.argtypes = [_p, _p, _p, ctypes.c_int, _i64, _i64, _i64, _i64, _i32, _i32,
                                          _p, _p, _p, _p, _i32, _i64, _i64, ctypes.c_int,
                                          _p, _p, _p, _p, _p, _p, _p]
        lib.lp_fp8_cast_e4m3.restype = ctypes.c_int
        lib.lp_fp8_cast_e4m3.argtypes = [_p, ctypes.c_int, _i64, _i64, _i64, _i32, _i32, _p, _p, _p]
        lib.lp_fp8_cast_current.restype = ctypes.c_int
        lib.lp_fp8_cast_current.argtypes = [_p, ctypes.c_int, _i64, _i64, _i64, _i32, _i32, _p, _p, _p, _p]
        lib.lp_fp8_cast_current_noalloc.restype = ctypes.c_int
        lib.lp_fp8_cast_current_noalloc.argtypes = [_p, ctypes.c_int, _i64, _i64, _i64, _i32, _i32, _p, _p, _p]
        lib.lp_attn_varlen_fwd.restype = ctypes.c_int
        lib.lp_attn_varlen_fwd.argtypes = [ctypes.POINTER(AttnArgs), _p]
        lib.lp_attn_varlen_bwd.restype = ctypes.c_int
        lib.lp_attn_varlen_bwd.argtypes = [ctypes.POINTER(BwdArgs), _p]
        _lib = lib
        return lib


def check(name: str, rc: int) -> None:
    if rc != LPFA_OK:
        msg = load().lpfa_last_error().decode(errors="replace")
        raise LpfaError(name, rc, msg)
