"""CPU oracle for the MXFP8 attention forward path — TEST INFRASTRUCTURE ONLY.

Plain, slow, obviously-correct NumPy (float64) code that states what the GPU path
computes. Only the test suite, the smoke check and the benchmark's CPU-baseline leg
may import it; the product path (the HIP library and its Python binding) never does,
and the oracle imports nothing from the product path. The two share no code; the
only module both sides use is ``synth`` (seeded input draws, no method arithmetic).

Sources (the pages this project follows):

* "LP-FA4" README (facebookresearch ads_model_kernel_library), section "MXFP8
  forward and backward": packed (tokens, heads, 128) inputs, E4M3 payloads with
  one E8M0 scale per 32-element block, per-sequence 128-token-padded scale
  storage, RCEIL default and FLOOR option, forward returns (out, lse); its
  introduction: noncausal head_dim-128 MHA, dense attention as uniform packed
  offsets.
* FastVideo PR "[feat]: fp8 PV mode for the FA4-FP4 attention path": the fp8 PV
  mode casts V to E4M3 with no scale factors (implicit dequant scale 1.0) and
  the output stays BF16; the bf16 mode keeps V in BF16.
* vLLM PR "FA4: no FP8 descale for a unit per-tensor scale": per-tensor q/k/v
  descales; a missing descale reads as 1.0, so a unit descale is bit-identical
  to none, and a descale of 2 changes the output.
* TensorRT-LLM PR "TE FP8 attention backend for VisualGen": Q/K/V and O scales
  written from the current tensors before every call (per-tensor current scaling).
* The same LP-FA4 README section for the backward: quantized Q/K/V in both hardware
  orientations, the forward's output and LSE, dQ in BF16 and dK/dV in BF16 or MXFP8.

Readings taken where the pages are silent are stated in each function.

Parity status: every function here is pinned by the ``-m "not gpu"`` tests
(closed forms, hand-computed encodings, a library cross-check of the E4M3
encoder, brute force on tiny shapes); none is "parity unpinned".
"""
from .fp8 import (E4M3_MAX, E4M3_VALUES, e4m3_decode, e4m3_encode, e8m0_decode,
                  bf16_round, bf16_encode)
from .mx import (padded_len, scale_offsets, mx_block_exponent, mx_quantize_varlen,
                 mx_dequantize_varlen, mx_quantize_varlen_tokens, mx_dequantize_varlen_tokens,
                 e4m3_cast, pertensor_quantize)
from .attention import attention_varlen, AttentionResult
from .current import current_scale, current_quantize
from .backward import attention_varlen_bwd, BackwardResult

__all__ = [
    "E4M3_MAX", "E4M3_VALUES", "e4m3_decode", "e4m3_encode", "e8m0_decode", "bf16_round",
    "bf16_encode", "padded_len", "scale_offsets", "mx_block_exponent", "mx_quantize_varlen",
    "mx_dequantize_varlen", "mx_quantize_varlen_tokens", "mx_dequantize_varlen_tokens", "e4m3_cast", "pertensor_quantize", "attention_varlen",
    "AttentionResult", "current_scale", "current_quantize", "attention_varlen_bwd", "BackwardResult",
]
