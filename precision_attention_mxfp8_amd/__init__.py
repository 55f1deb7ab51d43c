"""MXFP8 attention forward for AMD Instinct MI355X (gfx950): HIP kernels behind a C ABI.

Public API (marshalling only; the work runs in liblpfa.so):
  VarlenMeta.from_lengths, quantize_mxfp8_varlen, quantize_mxfp8_varlen_tokens, cast_e4m3,
  prepare_qkv (quantize Q, K and cast V in one launch),
  cast_e4m3_current (per-tensor current scaling), cast_e4m3_current_noalloc (the same with no
  allocation: scratch in a static device array),
  lp_attn_varlen_fwd, AttnPlan (a prepared lp_attn_varlen_fwd for repeated calls),
  lp_attn_varlen_bwd (gradients on MXFP8 operands; dK/dV in BF16 or MXFP8), BwdPlan (prepared),
  longest_first_tile_order.
"""
from .api import (AttnPlan, BwdPlan, Mxfp8Tensor, Mxfp8TokensTensor, VarlenMeta, cast_e4m3, cast_e4m3_current,
                  cast_e4m3_current_noalloc,
                  e4m3_group_max_shape, longest_first_tile_order,
                  lp_attn_varlen_bwd, lp_attn_varlen_fwd, prepare_qkv, quantize_mxfp8_varlen,
                  quantize_mxfp8_varlen_tokens)
from ._lib import LpfaError, load as load_library

__all__ = ["AttnPlan", "BwdPlan", "Mxfp8Tensor", "Mxfp8TokensTensor", "VarlenMeta", "cast_e4m3", "cast_e4m3_current",
           "cast_e4m3_current_noalloc",
           "e4m3_group_max_shape", "longest_first_tile_order",
           "lp_attn_varlen_bwd", "lp_attn_varlen_fwd", "prepare_qkv", "quantize_mxfp8_varlen", "quantize_mxfp8_varlen_tokens", "LpfaError",
           "load_library"]
