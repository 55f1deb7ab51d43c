// Host-side argument checks (see validate.h). The rules restate the contract of include/lpfa.h.
#include "validate.h"

#include <climits>
#include <cmath>
#include <cstddef>
#include <cstdint>
#include <cstring>
#include <sstream>

namespace lpfa {

namespace {
thread_local std::string g_error;

int fail(int code, const std::string& msg) {
  set_error(msg);
  return code;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// A strided (tokens, heads, 128) input: pointer and strides (in elements of `esize` bytes)
// must be 16-byte multiples so the kernels can use 16-byte loads.
int check_rows(const char* name, const void* p, int64_t stride_tok, int64_t stride_head,
               int64_t tokens, int32_t heads, int esize) {
  if (tokens == 0 || heads == 0) return LPFA_OK;
  if (p == nullptr) return fail(LPFA_EINVAL, std::string(name) + " is NULL");
  if (!aligned16(p)) return fail(LPFA_EINVAL, std::string(name) + " is not 16-byte aligned");
  if (stride_tok < 0 || stride_head < 0)
    return fail(LPFA_EINVAL, std::string(name) + " has a negative stride");
  if ((stride_tok * esize) % 16 != 0 || (stride_head * esize) % 16 != 0)
    return fail(LPFA_EINVAL, std::string(name) + " strides are not 16-byte multiples");
  if (heads > 1 && stride_head < 128)
    return fail(LPFA_EINVAL, std::string(name) + " head stride overlaps head_dim");
  if (tokens > 1 && stride_tok < 128)
    return fail(LPFA_EINVAL, std::string(name) + " token stride overlaps head_dim");
  return LPFA_OK;
}

int check_dtype(int x_dtype) {
  if (x_dtype != LPFA_DTYPE_BF16 && x_dtype != LPFA_DTYPE_FP32)
    return fail(LPFA_EINVAL, "x_dtype must be LPFA_DTYPE_BF16 or LPFA_DTYPE_FP32");
  return LPFA_OK;
}

int check_descale(const char* name, const float* p, int64_t s_seq, int64_t s_head) {
  if (p == nullptr) return LPFA_OK;
  if ((reinterpret_cast<uintptr_t>(p) & 3u) != 0) return fail(LPFA_EINVAL, std::string(name) + " is misaligned");
  if (s_seq < 0 || s_head < 0) return fail(LPFA_EINVAL, std::string(name) + " has a negative stride");
  return LPFA_OK;
}
}  // namespace

void set_error(const std::string& msg) { g_error = msg; }
void clear_error() { g_error.clear(); }
const char* last_error() { return g_error.c_str(); }

int check_quantize(const void* x, int x_dtype, int64_t stride_tok, int64_t stride_head,
                   int64_t total_tokens, int32_t num_heads, int32_t head_dim,
                   const int32_t* cu_seqlens, const int32_t* cu_scale, int32_t num_seqs,
                   int64_t total_scale_rows, int scaling_mode, const uint8_t* payload,
                   const uint8_t* scales) {
  if (int rc = check_dtype(x_dtype)) return rc;
  if (scaling_mode != LPFA_SCALING_RCEIL && scaling_mode != LPFA_SCALING_FLOOR)
    return fail(LPFA_EINVAL, "scaling_mode must be LPFA_SCALING_RCEIL or LPFA_SCALING_FLOOR");
  if (head_dim != 128) return fail(LPFA_ENOTSUP, "head_dim must be 128");
  if (total_tokens < 0 || num_heads < 1 || num_seqs < 0 || total_scale_rows < 0)
    return fail(LPFA_EINVAL, "negative size, or num_heads < 1");
  if (total_scale_rows < total_tokens)
    return fail(LPFA_EINVAL, "total_scale_rows is smaller than total_tokens");
  if (total_scale_rows % 128 != 0)
    return fail(LPFA_EINVAL, "total_scale_rows must be a multiple of 128 (per-sequence padding)");
  if (total_scale_rows > 0 && num_seqs == 0)
    return fail(LPFA_EINVAL, "scale rows without sequences");
  if (total_scale_rows * (int64_t)num_heads > (int64_t)INT32_MAX * 16)
    return fail(LPFA_ENOTSUP, "tensor too large for one launch");
  if (num_seqs > 0 && (cu_seqlens == nullptr || cu_scale == nullptr))
    return fail(LPFA_EINVAL, "cu_seqlens / cu_scale is NULL");
  int esize = x_dtype == LPFA_DTYPE_BF16 ? 2 : 4;
  if (int rc = check_rows("x", x, stride_tok, stride_head, total_tokens, num_heads, esize)) return rc;
  if (total_tokens > 0 && payload == nullptr) return fail(LPFA_EINVAL, "payload is NULL");
  if (total_scale_rows > 0 && scales == nullptr) return fail(LPFA_EINVAL, "scales is NULL");
  if (payload && !aligned16(payload)) return fail(LPFA_EINVAL, "payload is not 16-byte aligned");
  if (scales && (reinterpret_cast<uintptr_t>(scales) & 3u))
    return fail(LPFA_EINVAL, "scales is not 4-byte aligned");
  clear_error();
  return LPFA_OK;
}

int check_cast(const void* x, int x_dtype, int64_t stride_tok, int64_t stride_head,
               int64_t total_tokens, int32_t num_heads, int32_t head_dim, const uint8_t* y) {
  if (int rc = check_dtype(x_dtype)) return rc;
  if (head_dim != 128) return fail(LPFA_ENOTSUP, "head_dim must be 128");
  if (total_tokens < 0 || num_heads < 1) return fail(LPFA_EINVAL, "negative size, or num_heads < 1");
  if (total_tokens * (int64_t)num_heads > (int64_t)INT32_MAX * 16)
    return fail(LPFA_ENOTSUP, "tensor too large for one launch");
  int esize = x_dtype == LPFA_DTYPE_BF16 ? 2 : 4;
  if (int rc = check_rows("x", x, stride_tok, stride_head, total_tokens, num_heads, esize)) return rc;
  if (total_tokens > 0 && y == nullptr) return fail(LPFA_EINVAL, "y is NULL");
  if (y && !aligned16(y)) return fail(LPFA_EINVAL, "y is not 16-byte aligned");
  clear_error();
  return LPFA_OK;
}

// Float classification from the bits: the library is compiled with -fno-honor-nans (the kernels'
// inputs are finite by contract), under which std::isnan / std::isfinite may fold to constants,
// but host arguments still have to be checked for NaN and infinity.
static bool float_is_nan(float f) {
  uint32_t b;
  std::memcpy(&b, &f, sizeof b);
  return (b & 0x7FFFFFFFu) > 0x7F800000u;
}

static bool float_finite_positive(float f) {
  uint32_t b;
  std::memcpy(&b, &f, sizeof b);
  return (b >> 31) == 0 && (b & 0x7F800000u) != 0x7F800000u && b != 0;
}

int check_attn(const lpfa_attn_args* a) {
  if (a == nullptr) return fail(LPFA_EINVAL, "args is NULL");
  if (a->struct_size < (int32_t)sizeof(lpfa_attn_args))
    return fail(LPFA_EINVAL, "struct_size is smaller than this library's lpfa_attn_args");
  if (a->head_dim != 128) return fail(LPFA_ENOTSUP, "head_dim must be 128");
  if (a->causal != 0) return fail(LPFA_ENOTSUP, "only noncausal attention is implemented");
  if (a->pv_mode != LPFA_PV_BF16 && a->pv_mode != LPFA_PV_FP8 && a->pv_mode != LPFA_PV_MX)
    return fail(LPFA_EINVAL, "pv_mode must be LPFA_PV_BF16, LPFA_PV_FP8 or LPFA_PV_MX");
  if ((a->pv_mode == LPFA_PV_MX) != (a->v_scale != nullptr))
    return fail(LPFA_EINVAL, "v_scale is required in the LPFA_PV_MX mode and must be NULL otherwise");
  if (a->qk_bf16 != 0 && a->qk_bf16 != 1) return fail(LPFA_EINVAL, "qk_bf16 must be 0 or 1");
  if (a->qk_bf16 && (a->q_scale != nullptr || a->k_scale != nullptr))
    return fail(LPFA_EINVAL, "BF16 Q/K (qk_bf16) take no block scales");
  if (a->qk_bf16 && a->pv_mode != LPFA_PV_BF16)
    return fail(LPFA_EINVAL, "BF16 Q/K (qk_bf16) need BF16 V (pv_mode LPFA_PV_BF16)");
  if (a->pv_mode == LPFA_PV_MX && a->q_scale == nullptr)
    return fail(LPFA_EINVAL, "the LPFA_PV_MX mode needs MX Q and K (q_scale and k_scale)");
  if (a->v_scale && (reinterpret_cast<uintptr_t>(a->v_scale) & 3u))
    return fail(LPFA_EINVAL, "v_scale must be 4-byte aligned");
  if (a->num_seqs < 0 || a->num_heads < 1 || a->total_q < 0 || a->total_k < 0 ||
      a->max_seqlen_q < 0 || a->max_seqlen_k < 0)
    return fail(LPFA_EINVAL, "negative size, or num_heads < 1");
  if (!float_finite_positive(a->softmax_scale))
    return fail(LPFA_EINVAL, "softmax_scale must be finite and positive");
  if (float_is_nan(a->fp8_score_guard)) return fail(LPFA_EINVAL, "fp8_score_guard is NaN");
  if (a->k_deq && (a->q_scale == nullptr || a->k_scale == nullptr || a->pv_mode != LPFA_PV_BF16 || a->qk_bf16))
    return fail(LPFA_EINVAL, "k_deq needs MX Q and K (q_scale, k_scale) and pv_mode LPFA_PV_BF16");
  if (a->k_deq && !aligned16(a->k_deq)) return fail(LPFA_EINVAL, "k_deq is not 16-byte aligned");
  if ((a->q_scale == nullptr) != (a->k_scale == nullptr))
    return fail(LPFA_EINVAL, "q_scale and k_scale must both be set (MX mode) or both be NULL (per-tensor mode)");
  if (a->q_scale && (a->cu_scale_q == nullptr || a->cu_scale_k == nullptr))
    return fail(LPFA_EINVAL, "MX mode needs cu_scale_q and cu_scale_k");
  if (a->q_scale && ((reinterpret_cast<uintptr_t>(a->q_scale) & 3u) || (reinterpret_cast<uintptr_t>(a->k_scale) & 3u)))
    return fail(LPFA_EINVAL, "q_scale / k_scale must be 4-byte aligned");
  if (a->v_descale != nullptr && a->pv_mode == LPFA_PV_BF16)
    return fail(LPFA_EINVAL, "v_descale is only meaningful with FP8 V (pv_mode LPFA_PV_FP8 or LPFA_PV_MX)");
  if (a->num_seqs > 0 && (a->cu_seqlens_q == nullptr || a->cu_seqlens_k == nullptr))
    return fail(LPFA_EINVAL, "cu_seqlens_q / cu_seqlens_k is NULL");
  if (a->max_seqlen_q > a->total_q) return fail(LPFA_EINVAL, "max_seqlen_q exceeds total_q");
  if (a->max_seqlen_k > a->total_k) return fail(LPFA_EINVAL, "max_seqlen_k exceeds total_k");
  const int qksize = a->qk_bf16 ? 2 : 1;
  if (int rc = check_rows("q", a->q, a->q_stride_tok, a->q_stride_head, a->total_q, a->num_heads, qksize)) return rc;
  if (int rc = check_rows("k", a->k, a->k_stride_tok, a->k_stride_head, a->total_k, a->num_heads, qksize)) return rc;
  int vsize = a->pv_mode == LPFA_PV_BF16 ? 2 : 1;
  if (int rc = check_rows("v", a->v, a->v_stride_tok, a->v_stride_head, a->total_k, a->num_heads, vsize)) return rc;
  if (int rc = check_descale("q_descale", a->q_descale, a->q_descale_stride_seq, a->q_descale_stride_head)) return rc;
  if (int rc = check_descale("k_descale", a->k_descale, a->k_descale_stride_seq, a->k_descale_stride_head)) return rc;
  if (int rc = check_descale("v_descale", a->v_descale, a->v_descale_stride_seq, a->v_descale_stride_head)) return rc;
  if (a->total_q > 0 && (a->out == nullptr || a->lse == nullptr)) return fail(LPFA_EINVAL, "out / lse is NULL");
  if (a->out && !aligned16(a->out)) return fail(LPFA_EINVAL, "out is not 16-byte aligned");
  if (a->lse && (reinterpret_cast<uintptr_t>(a->lse) & 3u)) return fail(LPFA_EINVAL, "lse is misaligned");
  if (a->tile_order != nullptr && a->num_tiles < 0) return fail(LPFA_EINVAL, "num_tiles is negative");
  if (a->tile_order == nullptr && a->num_tiles != 0)
    return fail(LPFA_EINVAL, "num_tiles given without tile_order");
  int64_t qtiles = ((int64_t)a->max_seqlen_q + 127) / 128;
  if ((int64_t)a->num_seqs * a->num_heads * qtiles > INT32_MAX)
    return fail(LPFA_ENOTSUP, "too many work tiles for one launch");
  if (a->total_q * (int64_t)a->num_heads > INT32_MAX || a->total_k * (int64_t)a->num_heads > (int64_t)INT32_MAX * 8)
    return fail(LPFA_ENOTSUP, "tensor too large for one launch");
  clear_error();
  return LPFA_OK;
}

int check_bwd(const lpfa_bwd_args* a) {
  clear_error();
  if (a == nullptr) return fail(LPFA_EINVAL, "args is NULL");
  if (a->struct_size < (int32_t)sizeof(lpfa_bwd_args))
    return fail(LPFA_EINVAL, "struct_size is smaller than this library's lpfa_bwd_args");
  if (a->head_dim != 128) return fail(LPFA_ENOTSUP, "head_dim must be 128");
  if (a->causal != 0) return fail(LPFA_ENOTSUP, "only noncausal attention is implemented");
  if (a->num_seqs < 0 || a->num_heads < 1 || a->total_q < 0 || a->total_k < 0 || a->total_scale_rows_q < 0 ||
      a->total_scale_rows_k < 0)
    return fail(LPFA_EINVAL, "negative size, or num_heads < 1");
  if (a->total_scale_rows_q % 128 != 0 || a->total_scale_rows_k % 128 != 0)
    return fail(LPFA_EINVAL, "total scale rows must be multiples of 128");
  if (a->total_scale_rows_q < a->total_q || a->total_scale_rows_k < a->total_k)
    return fail(LPFA_EINVAL, "total scale rows below the token count");
  if (!float_finite_positive(a->softmax_scale))
    return fail(LPFA_EINVAL, "softmax_scale must be finite and positive");
  if (a->output_mxfp8_dkv != 0 && a->output_mxfp8_dkv != 1) return fail(LPFA_EINVAL, "output_mxfp8_dkv must be 0 or 1");
  if (a->scaling_mode != LPFA_SCALING_RCEIL && a->scaling_mode != LPFA_SCALING_FLOOR)
    return fail(LPFA_EINVAL, "scaling_mode must be RCEIL or FLOOR");
  if ((a->dk_scale != nullptr || a->dv_scale != nullptr) != (a->output_mxfp8_dkv != 0) ||
      (a->output_mxfp8_dkv && (a->dk_scale == nullptr || a->dv_scale == nullptr)))
    return fail(LPFA_EINVAL, "dk_scale and dv_scale are required with output_mxfp8_dkv and rejected without");
  if (a->num_seqs > 0 && (a->cu_seqlens_q == nullptr || a->cu_seqlens_k == nullptr || a->cu_scale_q == nullptr ||
                          a->cu_scale_k == nullptr))
    return fail(LPFA_EINVAL, "cu_seqlens / cu_scale is NULL");
  if (a->num_seqs == 0 && (a->total_q != 0 || a->total_k != 0))
    return fail(LPFA_EINVAL, "tokens without sequences");
  struct Need {
    const void* ptr;
    bool used;
    const char* name;
    unsigned align;
  };
  const bool hq = a->total_q > 0, hk = a->total_k > 0, both = hq && hk;
  const Need need[] = {
      {a->q, both, "q", 16u},           {a->q_scale, both, "q_scale", 1u},
      {a->k, both, "k", 16u},           {a->k_scale, both, "k_scale", 1u},
      {a->v, both, "v", 16u},           {a->v_scale, both, "v_scale", 1u},
      {a->q_t, both, "q_t", 16u},       {a->q_t_scale, both, "q_t_scale", 16u},
      {a->k_t, both, "k_t", 16u},       {a->k_t_scale, both, "k_t_scale", 16u},
      {a->out, hq, "out", 16u},         {a->dout, hq, "dout", 16u},
      {a->lse, both, "lse", 4u},        {a->work, hq || hk, "work", 256u},
      {a->dq, hq, "dq", 16u},           {a->dk, hk, "dk", 16u},
      {a->dv, hk, "dv", 16u},
  };
  for (const Need& n : need) {
    if (!n.used) continue;
    if (n.ptr == nullptr) return fail(LPFA_EINVAL, std::string(n.name) + " is NULL");
    if ((reinterpret_cast<uintptr_t>(n.ptr) & (n.align - 1u)) != 0)
      return fail(LPFA_EINVAL, std::string(n.name) + " is misaligned");
  }
  if ((a->total_q + 1) * (int64_t)a->num_heads * 128 * 4 > INT64_MAX / 4 ||
      a->total_scale_rows_q / 64 > 0x7FFFFFFF || a->total_scale_rows_k / 64 > 0x7FFFFFFF ||
      (a->total_q * (int64_t)a->num_heads * 16 + 255) / 256 > 0x7FFFFFFF)
    return fail(LPFA_ENOTSUP, "tensor too large for one launch");
  if (a->num_heads > 65535) return fail(LPFA_ENOTSUP, "num_heads above the launch grid's limit");
  return LPFA_OK;
}

}  // namespace lpfa
