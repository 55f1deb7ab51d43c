/*
 * lpfa.h - C ABI of the MXFP8 attention library for AMD Instinct MI355X (gfx950).
 *
 * The library does these things, all on the GPU, all on a stream the caller owns:
 *   1. MXFP8 quantization of packed variable-length (tokens, heads, 128) tensors:
 *      E4M3 payloads plus one E8M0 scale per 32-element block along head_dim, each
 *      sequence with its own scale storage padded to a multiple of 128 tokens
 *      (LP-FA4 README, section "MXFP8 forward and backward"), and the unscaled E4M3
 *      cast of V used by the fp8 PV mode (FastVideo PR "fp8 PV mode for the FA4-FP4
 *      attention path", description of the fa4_v_to_fp8 op).
 *   2. A fused noncausal head_dim-128 attention forward over packed sequences
 *      (LP-FA4 README, introduction: dense attention is uniform packed offsets),
 *      S = Q K^T on block-scaled E4M3 operands, online softmax, then P V with V in
 *      BF16 or unscaled E4M3, writing O in BF16 and the log-sum-exp in FP32.
 *      Optional per-tensor q/k/v descales; a missing descale is read as 1.0 with the
 *      same arithmetic, so a unit descale gives bit-identical output (vLLM PR
 *      "FA4: no FP8 descale for a unit per-tensor scale", sections "Claims" and
 *      "Validation"). Variants: V MXFP8 along tokens (the second hardware
 *      orientation), and BF16 Q/K (the BF16 FlashAttention forward, for comparison).
 *   3. The backward of that attention on MXFP8 operands in both orientations: dQ in
 *      BF16, dK and dV in BF16 or MXFP8 (LP-FA4 README, same section).
 *   4. Per-tensor current scaling to E4M3 (TensorRT-LLM PR "TE FP8 attention backend for
 *      VisualGen", inference scaling fix), and the forward's three preparation passes
 *      (quantize Q and K, cast V) in one launch.
 *
 * Conventions for every entry point
 *   - All tensor arguments are DEVICE pointers to memory the caller allocated (two
 *     entry points also take a caller-owned workspace; lp_fp8_cast_current_noalloc keeps
 *     its scratch in a static device array instead); the
 *     library never allocates, frees or synchronises, and launches only on `stream`
 *     (a hipStream_t passed as void*; NULL means the default stream).
 *   - Strides are in elements. Element types: BF16 = raw uint16 bit patterns,
 *     E4M3 / E8M0 = uint8 codes, FP32 = float.
 *   - Return value: LPFA_OK (0) or a negative code. On error nothing is launched,
 *     and lpfa_last_error() describes the problem. All argument checks run on the
 *     host and read no device memory; device-resident offsets (cu_seqlens, cu_scale)
 *     are trusted, so their consistency is the caller's duty.
 *   - Launch failures return LPFA_EIO; faults inside a kernel surface at the
 *     caller's next synchronisation, as for any asynchronous launch.
 *   - Entry points are thread-safe; concurrent calls on different streams do not
 *     share state.
 *   - With LPFA_LOG=1 in the environment, the first lp_attn_varlen_fwd call of each variant
 *     in the process prints one line to stderr naming the Q/K and V types fed to the kernel
 *     (FastVideo fp8-PV PR: a once-per-process log of the V dtype the attention received).
 */
#ifndef LPFA_H
#define LPFA_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define LPFA_ABI_VERSION 9

#define LPFA_OK 0
#define LPFA_EIO (-5)      /* kernel launch failed */
#define LPFA_EINVAL (-22)  /* bad pointer, size, stride, alignment or enum value */
#define LPFA_ENOTSUP (-95) /* well-formed but outside what the kernels implement */

#define LPFA_DTYPE_BF16 0
#define LPFA_DTYPE_FP32 1

#define LPFA_SCALING_RCEIL 0 /* default: smallest e with amax <= 448 * 2^e */
#define LPFA_SCALING_FLOOR 1 /* e = floor(log2 amax) - 8 */

#define LPFA_PV_BF16 0 /* V is BF16 (default mode, behaviour unchanged) */
#define LPFA_PV_FP8 1  /* V is unscaled E4M3, implicit dequant scale 1.0 */
#define LPFA_PV_MX 2   /* V is MXFP8 along tokens (mxfp8_quantize_varlen_tokens); P unscaled E4M3 */

/* Version of this ABI (LPFA_ABI_VERSION of the built library). */
int lpfa_abi_version(void);

/* Message of the last error returned on the calling thread ("" if none). The pointer
 * stays valid until the next call on the same thread. */
const char* lpfa_last_error(void);

/*
 * mxfp8_quantize_varlen - MXFP8 quantization of a packed varlen tensor.
 * (LP-FA4 README, section "MXFP8 forward and backward": E4M3 payload with one E8M0
 *  scale per 32 elements, per-sequence 128-token-padded scale storage, RCEIL default,
 *  FLOOR optional.)
 *
 * For every token t of sequence i, head h and 32-element block b of head_dim:
 *   amax = max |x| over the block; e = RCEIL or FLOOR exponent of amax, clamped to
 *   [-127, 127] (e = -127 for an all-zero block); scales[row, h, b] = e + 127;
 *   payload[t, h, 32b + j] = E4M3(x * 2^-e) rounded to nearest even, saturating at 448.
 *   row = cu_scale[i] + (t - cu_seqlens[i]).
 * Scale rows from L_i to P(L_i)-1 of each sequence (P(L) = L rounded up to a multiple
 * of 128) are pad rows and are written as 0x7F.
 *
 *   x            input, x[t * stride_tok + h * stride_head + d], d = 0..127 contiguous.
 *                BF16 or FP32 (x_dtype). x and both strides times the element size
 *                must be multiples of 16 bytes. Values must be finite.
 *   total_tokens T = cu_seqlens[num_seqs]; num_heads >= 1; head_dim must be 128.
 *   cu_seqlens   device int32[num_seqs + 1], 0 = cu_seqlens[0] <= ... (packed offsets).
 *   cu_scale     device int32[num_seqs + 1], prefix sums of P(L_i).
 *   total_scale_rows  cu_scale[num_seqs].
 *   payload      output uint8 (T, num_heads, 128), contiguous.
 *   scales       output uint8 (total_scale_rows, num_heads, 4), contiguous.
 *   group_max    optional output (NULL: not written) uint8 (total_scale_rows / 16, num_heads):
 *                entry [k, h] is the largest scale byte of head h over the rows of 16-row group
 *                k (rows 16k .. 16k+15) that are not pad rows, 0 if all of them are. Passed to
 *                lp_attn_varlen_fwd as k_scale_group_max for K, it replaces the attention
 *                kernel's scan of the K scales (same results).
 *   deq          optional output (NULL: not written) BF16 (T, num_heads, 128), contiguous,
 *                16-byte aligned: the quantized values themselves, payload * 2^e, converted to
 *                BF16 exactly as the attention's guarded path converts them (one E4M3 code
 *                times a power of two has at most 4 significant bits). Passed to
 *                lp_attn_varlen_fwd as k_deq for K, it spares the tiles that fail the precision
 *                guard their own conversion of every K block (same results). 2 bytes per element
 *                more; a design choice for gfx950, whose FP8 accumulation needs the guard.
 * Errors: LPFA_EINVAL for NULL pointers (unless the tensor is empty), negative sizes,
 * misalignment, bad enum values; LPFA_ENOTSUP for head_dim != 128.
 */
int mxfp8_quantize_varlen(const void* x, int x_dtype, int64_t stride_tok, int64_t stride_head,
                          int64_t total_tokens, int32_t num_heads, int32_t head_dim,
                          const int32_t* cu_seqlens, const int32_t* cu_scale, int32_t num_seqs,
                          int64_t total_scale_rows, int scaling_mode, uint8_t* payload,
                          uint8_t* scales, uint8_t* group_max, uint16_t* deq, void* stream);

/*
 * mxfp8_quantize_varlen_tokens - MXFP8 quantization along tokens (the P V operand's V).
 * (LP-FA4 README, section "MXFP8 forward and backward": V is quantized like Q and K and
 *  keeps both hardware orientations; the P V product contracts over tokens, so its V
 *  operand takes blocks of 32 tokens.)
 *
 * For sequence i, head h, column d and 32-token block b of the sequence (tokens
 * cu_seqlens[i] + 32b .. + 32b + 31, the last block of a sequence holding its real tokens
 * only): amax = max |x| over the block's tokens; e, the scale byte e + 127 and
 * payload[t, h, d] = E4M3(x * 2^-e) follow the rules of mxfp8_quantize_varlen.
 *   scales[row, h, d] with row = cu_scale[i] / 32 + b; rows of a sequence past its last
 *   block (up to P(L_i) / 32) are written as 0x7F.
 *
 *   x, strides, total_tokens, num_heads, head_dim, cu_seqlens, cu_scale, total_scale_rows,
 *   scaling_mode: as in mxfp8_quantize_varlen (cu_scale: prefix sums of P(L_i)).
 *   payload      output uint8 (T, num_heads, 128), contiguous.
 *   scales       output uint8 (total_scale_rows / 32, num_heads, 128), contiguous.
 * Errors: as mxfp8_quantize_varlen.
 */
int mxfp8_quantize_varlen_tokens(const void* x, int x_dtype, int64_t stride_tok, int64_t stride_head,
                                 int64_t total_tokens, int32_t num_heads, int32_t head_dim,
                                 const int32_t* cu_seqlens, const int32_t* cu_scale, int32_t num_seqs,
                                 int64_t total_scale_rows, int scaling_mode, uint8_t* payload,
                                 uint8_t* scales, void* stream);

/*
 * lp_fp8_cast_e4m3 - unscaled E4M3 cast (the fp8 PV mode's V; per-tensor FP8 Q, K, V).
 * (FastVideo PR "fp8 PV mode for the FA4-FP4 attention path": an elementwise e4m3 cast
 *  of V with no scale factors; the attention reads it with dequant scale 1.0.)
 *
 *   y[t, h, d] = E4M3(x[t * stride_tok + h * stride_head + d]), nearest even,
 *   saturating finite values above 448 to +-448 (sign kept, so -0 and negative
 *   underflow give 0x80).
 *   x: BF16 or FP32, 16-byte aligned with 16-byte-multiple strides; y: uint8
 *   (total_tokens, num_heads, 128) contiguous. head_dim must be 128.
 *   group_max: optional output (NULL: not written, ABI 8) uint8 (ceil(total_tokens / 16),
 *   num_heads): entry [g, h] is the largest code magnitude (code & 0x7F) of head h over tokens
 *   16g .. 16g+15 (those that exist). Passed to lp_attn_varlen_fwd as k_scale_group_max for a
 *   per-tensor K, it gives the precision guard its bound on |k| (vLLM unit-descale PR: per-tensor
 *   FP8 attention; without it the guard must assume the E4M3 range, 448).
 */
int lp_fp8_cast_e4m3(const void* x, int x_dtype, int64_t stride_tok, int64_t stride_head,
                     int64_t total_tokens, int32_t num_heads, int32_t head_dim, uint8_t* y,
                     uint8_t* group_max, void* stream);

/*
 * mxfp8_prepare_qkv - the forward's three preparation passes in one launch: Q and K as
 * mxfp8_quantize_varlen (K with its group maxima) and V as lp_fp8_cast_e4m3 (the fp8 PV mode).
 * (LP-FA4 README, section "MXFP8 forward and backward"; FastVideo fp8-PV PR: unscaled V cast.)
 *
 * The outputs are byte-identical to the three separate calls; only the launch is shared. q, k
 * and v have one dtype (x_dtype) and the same token and head strides (elements); total_q and
 * total_k are their token counts (v has total_k). The metadata, payload, scale and group-max
 * arguments mean what they mean for mxfp8_quantize_varlen (k_group_max may be NULL); v_codes is
 * uint8 (total_k, num_heads, 128) contiguous.
 * Errors: those of the three separate calls.
 */
int mxfp8_prepare_qkv(const void* q, const void* k, const void* v, int x_dtype, int64_t stride_tok,
                      int64_t stride_head, int64_t total_q, int64_t total_k, int32_t num_heads,
                      int32_t head_dim, const int32_t* cu_seqlens_q, const int32_t* cu_scale_q,
                      const int32_t* cu_seqlens_k, const int32_t* cu_scale_k, int32_t num_seqs,
                      int64_t total_scale_rows_q, int64_t total_scale_rows_k, int scaling_mode,
                      uint8_t* q_payload, uint8_t* q_scales, uint8_t* k_payload, uint8_t* k_scales,
                      uint8_t* k_group_max, uint8_t* v_codes, void* stream);

/*
 * lp_fp8_cast_current - per-tensor current scaling to E4M3.
 * (TensorRT-LLM PR "TE FP8 attention backend for VisualGen": the Q/K/V and O scales are
 *  written from the current tensors before every call, so small tensors such as an attention
 *  output spread over many keys keep E4M3's normal range.)
 *
 *   amax = max |x| over the whole tensor; s = amax / 448 in float32 (s = 1 if amax = 0);
 *   descale[0] = s; y[t, h, d] = E4M3(x / s) with the quotient rounded to float32, nearest
 *   even, saturating at 448. x: BF16 or FP32 as in lp_fp8_cast_e4m3; y: uint8 (total_tokens,
 *   num_heads, 128) contiguous; descale: device float32, 4-byte aligned (the per-tensor q/k/v
 *   descale of lp_attn_varlen_fwd, strides 0); work: caller-owned device workspace of
 *   LPFA_CURRENT_WORK_FLOATS floats (partial maxima between the two kernels, no clearing
 *   needed); on completion work[0] = amax. Calls that share a work buffer on one stream run
 *   in order; concurrent calls need their own.
 * Errors: as lp_fp8_cast_e4m3, and LPFA_EINVAL for a NULL or misaligned work / descale.
 */
int lp_fp8_cast_current(const void* x, int x_dtype, int64_t stride_tok, int64_t stride_head,
                        int64_t total_tokens, int32_t num_heads, int32_t head_dim, float* work, uint8_t* y,
                        float* descale, void* stream);

/* Floats in lp_fp8_cast_current's workspace: amax, then one partial maximum per amax workgroup. */
#define LPFA_CURRENT_WORK_FLOATS 257

/*
 * lp_fp8_cast_current_noalloc - lp_fp8_cast_current without a workspace argument, for callers
 * that cannot allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc). Same arguments, results and errors as lp_fp8_cast_current
 * minus `work`: the partial maxima live in a static device array of the library (2 KB per GPU,
 * held until the process ends), which holds what every input size needs, so no size is rejected
 * for it. The call allocates nothing and needs no clearing (each call writes every partial
 * maximum it reads). All calls on one GPU share that array: calls that overlap on one GPU
 * (concurrent streams, or several threads) race and must be serialised by the caller.
 * Errors: those of lp_fp8_cast_current; LPFA_EIO if the array's device address cannot be
 * obtained.
 */
int lp_fp8_cast_current_noalloc(const void* x, int x_dtype, int64_t stride_tok, int64_t stride_head,
                                int64_t total_tokens, int32_t num_heads, int32_t head_dim, uint8_t* y,
                                float* descale, void* stream);

/* Default threshold of the attention's precision guard (lpfa_attn_args.fp8_score_guard). */
#define LPFA_FP8_SCORE_GUARD_DEFAULT 16.0f

/*
 * Arguments of lp_attn_varlen_fwd. Zero-initialise, then set struct_size =
 * sizeof(lpfa_attn_args); fields added by later ABI versions go at the end.
 */
typedef struct lpfa_attn_args {
  int32_t struct_size;

  /* Q and K: E4M3 payloads, (total_q | total_k, num_heads, 128) with token/head strides
   * in elements (head_dim contiguous; pointer and strides 16-byte multiples). */
  const uint8_t* q;
  const uint8_t* k;
  int64_t q_stride_tok, q_stride_head;
  int64_t k_stride_tok, k_stride_head;

  /* MX block scales, uint8 (cu_scale_*[num_seqs], num_heads, 4) contiguous. Both set:
   * block-scaled QK^T (the LP-FA4 MXFP8 forward). Both NULL: per-tensor FP8 mode
   * (every block scale reads as 1.0). One without the other is LPFA_EINVAL. */
  const uint8_t* q_scale;
  const uint8_t* k_scale;
  const int32_t* cu_scale_q; /* device int32[num_seqs + 1]; required with q_scale */
  const int32_t* cu_scale_k;

  /* V: BF16 (pv_mode LPFA_PV_BF16), E4M3 (LPFA_PV_FP8) or the E4M3 payload of
   * mxfp8_quantize_varlen_tokens (LPFA_PV_MX, with v_scale), (total_k, num_heads, 128). */
  const void* v;
  int64_t v_stride_tok, v_stride_head;
  int32_t pv_mode;

  /* Packed sequence offsets (device int32[num_seqs + 1]); queries of sequence r attend
   * to the keys of sequence r only. max_seqlen_q bounds every query length. */
  const int32_t* cu_seqlens_q;
  const int32_t* cu_seqlens_k;
  int32_t num_seqs;
  int32_t max_seqlen_q;
  int32_t max_seqlen_k;
  int64_t total_q;
  int64_t total_k;
  int32_t num_heads; /* queries and keys have the same head count (MHA) */
  int32_t head_dim;  /* must be 128 */

  /* Softmax scale on the scores (callers usually pass 1/sqrt(128)); must be finite, > 0. */
  float softmax_scale;
  int32_t causal; /* must be 0: only noncausal attention is implemented */

  /* Optional per-tensor descales, fp32, element [seq * stride_seq + head * stride_head]
   * (strides may be 0 for broadcast). NULL reads as 1.0 through the same arithmetic.
   * Scores are multiplied by q_descale * k_descale, O by v_descale. */
  const float* q_descale;
  const float* k_descale;
  const float* v_descale;
  int64_t q_descale_stride_seq, q_descale_stride_head;
  int64_t k_descale_stride_seq, k_descale_stride_head;
  int64_t v_descale_stride_seq, v_descale_stride_head;

  /* Outputs: O BF16 (total_q, num_heads, 128) contiguous; LSE fp32 (num_heads, total_q),
   * natural log of the sum of exp of the scaled scores. A sequence with queries but no
   * keys gets O = 0 and LSE = -inf. */
  uint16_t* out;
  float* lse;

  /* Optional work order: device int32[3 * num_tiles] triples (seq, head, q_tile) of
   * 128-query tiles, launched in this order (e.g. longest sequences first). NULL: every
   * (seq, head, tile) in a default order. Each triple must be listed at most once. */
  const int32_t* tile_order;
  int32_t num_tiles;

  /* Optional timing: hipEvent_t handles the caller created. When set, the attention
   * kernel's own dispatch records them at its start and end (hipExtLaunchKernel), so
   * their elapsed time is the kernel's duration with no launch gap. When no kernel is
   * launched (no query tiles) both are recorded on the stream back to back. */
  void* start_event;
  void* stop_event;

  /* Optional K maxima for the precision guard (which picks the FP8 or the BF16 score path of a
   * query tile, from bounds on |q| and |k|; see fp8_score_guard).
   * MX mode: the group_max output of mxfp8_quantize_varlen for K, uint8
   * (cu_scale_k[num_seqs] / 16, num_heads); the guard reads the K bound there instead of
   * scanning k_scale, and its decisions, and so the results, are the same either way.
   * Per-tensor mode (ABI 8): the group_max output of lp_fp8_cast_e4m3 for K, uint8
   * (ceil(total_k / 16), num_heads), per 16 packed tokens; the guard bounds |k| by the largest
   * code of the groups that hold a sequence's keys (instead of 448, which sends typical data
   * to the BF16 score path). Ignored with qk_bf16. */
  const uint8_t* k_scale_group_max;

  /* LPFA_PV_MX only (required there, else must be NULL): V's token-block scales from
   * mxfp8_quantize_varlen_tokens, uint8 (cu_scale_k[num_seqs] / 32, num_heads, 128)
   * contiguous; needs the MX mode (q_scale and k_scale set). */
  const uint8_t* v_scale;

  /* 1: the BF16 FlashAttention forward (LP-FA4 README, the BF16 flash_attn_func path): q and k
   * point to BF16 (total, num_heads, 128) tensors (strides in elements, 16-byte multiples as
   * bytes), scores are BF16 products summed in FP32, and pv_mode must be LPFA_PV_BF16; q_scale
   * and k_scale must be NULL (q/k descales still apply). 0: E4M3 q and k as above. */
  int32_t qk_bf16;

  /* Threshold of the precision guard (ABI 8). A query tile computes its scores with the FP8
   * matrix instruction when c * max|q| * max|k| <= fp8_score_guard, with c = softmax_scale *
   * log2(e) * qd * kd and the bounds taken from the block scales (MX mode) or the codes and
   * k_scale_group_max (per-tensor mode); otherwise with BF16 products of the exactly
   * dequantized operands. The FP8 instruction truncates each product toward zero onto a grid 13
   * bits below the largest exponent sum of its group of 8, so FP8 scores err by at most about
   * 0.0137 * fp8_score_guard in log2 units (random-sign data by far less). 0 selects
   * LPFA_FP8_SCORE_GUARD_DEFAULT; a negative value never takes FP8 scores; NaN is LPFA_EINVAL. */
  float fp8_score_guard;

  /* Optional (ABI 9; NULL: none): K's quantized values as BF16, (total_k, num_heads, 128)
   * contiguous and 16-byte aligned, as mxfp8_quantize_varlen writes them into its deq output.
   * Tiles that fail the precision guard then load their K blocks from it instead of converting
   * every block of the payload themselves; results are identical either way. MX mode (q_scale
   * and k_scale set) with pv_mode LPFA_PV_BF16 only, else LPFA_EINVAL. */
  const void* k_deq;
} lpfa_attn_args;

/*
 * lp_attn_varlen_fwd - fused noncausal attention forward over packed sequences.
 * (LP-FA4 README, sections "MXFP8 forward and backward" and introduction; FastVideo
 *  fp8-PV PR; vLLM unit-descale PR.)
 *
 * For sequence r, head h, query i and key j:
 *   s_ij = softmax_scale * qd * kd * sum_b 2^(eq_ib + ek_jb) * sum_{d in b} q_id k_jd
 *   (eq, ek = 0 in per-tensor mode; q, k the BF16 values with qk_bf16), running row max m and sum l over key blocks
 *   (online softmax), P rounded to V's type (BF16, or E4M3 with no scale), O_i =
 *   vd * (sum_j P_ij V_j) / l_i rounded to BF16, LSE_i = ln sum_j exp(s_ij). In the
 *   LPFA_PV_MX mode V_j = payload_j * 2^(ev) with ev the scale of token j's 32-token
 *   block in each column.
 * Errors: LPFA_EINVAL (NULL pointers, bad strides/alignment, scale presence mismatch,
 * v_descale with BF16 V, bad pv_mode, v_scale missing in (or given outside) the
 * LPFA_PV_MX mode or without q_scale/k_scale, qk_bf16 with block scales or with V not BF16,
 * struct_size too small, non-positive scale);
 * LPFA_ENOTSUP (head_dim != 128, causal != 0); LPFA_EIO (launch failure).
 */
int lp_attn_varlen_fwd(const lpfa_attn_args* args, void* stream);

/*
 * lp_attn_varlen_bwd - noncausal varlen attention backward on MXFP8 operands.
 * (LP-FA4 README, section "MXFP8 forward and backward": the backward takes the quantized Q, K,
 *  V, each kept in both hardware orientations, the forward's output and LSE and the output
 *  gradient; it returns dQ in BF16 and dK, dV in BF16 or, with output_mxfp8_dkv, as E4M3
 *  payloads with one E8M0 scale per 32-element block.)
 *
 * With tau = softmax_scale, per sequence r (its queries attend to its keys only) and head:
 *   P = exp(tau Qd Kd^T - LSE), dP = dO Vd^T, D = rowsum(dO * O), dS = P * (dP - D),
 *   dV = P^T dO, dK = tau dS^T Qt, dQ = tau dS Kt,
 * with Qd, Kd, Vd the head_dim-orientation operands (mxfp8_quantize_varlen) and Qt, Kt the
 * token-orientation ones (mxfp8_quantize_varlen_tokens): each product takes the orientation whose
 * blocks run along its contraction. The matrix products take P and dS rounded to BF16 (nearest
 * even) and the operands dequantized exactly into BF16; sums are FP32.
 *
 * All tensors are device memory, contiguous, owned by the caller:
 *   q, k, v          uint8 E4M3 (total_q | total_k, num_heads, 128); 16-byte aligned
 *   q_scale, ...     uint8 E8M0 (total_scale_rows_q | _k, num_heads, 4), the quantizer's layout
 *   q_t, k_t         uint8 E4M3 (total, num_heads, 128), token orientation; 16-byte aligned
 *   q_t_scale, ...   uint8 E8M0 (total_scale_rows / 32, num_heads, 128); 16-byte aligned
 *   out, dout        BF16 (total_q, num_heads, 128): the forward's output and its gradient
 *   lse              float32 (num_heads, total_q), natural log, from lp_attn_varlen_fwd
 *   work             device workspace of LPFA_BWD_WORK_BYTES(total_q, total_k, num_heads)
 *                    bytes, 256-byte aligned, overwritten: D above (float32 (num_heads,
 *                    total_q)), then BF16 copies of Qd, Qt, Kd, Vd, Kt dequantized once so the
 *                    main kernels stream plain BF16 tiles
 *   dq               BF16 (total_q, num_heads, 128), written
 *   dk, dv           BF16 (total_k, num_heads, 128), or with output_mxfp8_dkv = 1 uint8 E4M3
 *                    payloads of that shape plus dk_scale, dv_scale: uint8 E8M0
 *                    (total_scale_rows_k, num_heads, 4) laid out as mxfp8_quantize_varlen's
 *                    output (scaling_mode RCEIL or FLOOR; pad rows 0x7F)
 * The cu_* arrays are the forward's (int32, num_seqs + 1 entries). A sequence with queries
 * must have keys (its contents are trusted, as in the forward); one with keys but no queries
 * gets zero dK and dV. dq, dk and dv are deterministic: no atomics.
 * Errors: LPFA_EINVAL for a NULL or misaligned pointer, a bad size, enum or struct_size, or
 * scales given (or missing) against output_mxfp8_dkv; LPFA_ENOTSUP for head_dim != 128 or
 * causal; LPFA_EIO when a launch fails.
 */
typedef struct lpfa_bwd_args {
  int32_t struct_size;
  const uint8_t* q;
  const uint8_t* q_scale;
  const uint8_t* k;
  const uint8_t* k_scale;
  const uint8_t* v;
  const uint8_t* v_scale;
  const uint8_t* q_t;
  const uint8_t* q_t_scale;
  const uint8_t* k_t;
  const uint8_t* k_t_scale;
  const void* out;
  const void* dout;
  const float* lse;
  const int32_t* cu_seqlens_q;
  const int32_t* cu_seqlens_k;
  const int32_t* cu_scale_q;
  const int32_t* cu_scale_k;
  int32_t num_seqs;
  int32_t num_heads;
  int32_t head_dim;
  int32_t causal;
  int64_t total_q;
  int64_t total_k;
  int64_t total_scale_rows_q;
  int64_t total_scale_rows_k;
  float softmax_scale;
  int32_t output_mxfp8_dkv;
  int32_t scaling_mode;
  void* work;
  void* dq;
  void* dk;
  void* dv;
  uint8_t* dk_scale;
  uint8_t* dv_scale;
} lpfa_bwd_args;

/* Workspace bytes of lp_attn_varlen_bwd: D rounded up to 256 bytes, then five BF16 copies. */
#define LPFA_BWD_WORK_BYTES(total_q, total_k, num_heads)                                   \
  ((((int64_t)(num_heads) * (int64_t)(total_q) * 4 + 255) / 256) * 256 +                  \
   (int64_t)(num_heads) * 256 * (2 * (int64_t)(total_q) + 3 * (int64_t)(total_k)))

int lp_attn_varlen_bwd(const lpfa_bwd_args* args, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* LPFA_H */
