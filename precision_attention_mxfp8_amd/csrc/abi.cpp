// C ABI entry points (include/lpfa.h): host checks, then one launch on the caller's stream.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <string>

#include "kernels.h"
#include "lpfa.h"
#include "validate.h"

namespace {

int launch_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return LPFA_OK;
  lpfa::set_error(std::string(what) + " launch failed: " + hipGetErrorString(e));
  return LPFA_EIO;
}

// With LPFA_LOG=1 in the environment, the first launch of each forward variant in the process
// prints one line to stderr naming the operand types actually fed to the kernel (FastVideo fp8-PV
// PR: a once-per-process log of the V dtype that reached the attention kernel).
void log_variant_once(const lpfa_attn_args* a) {
  static const bool on = [] {
    const char* e = std::getenv("LPFA_LOG");
    return e != nullptr && e[0] == '1';
  }();
  if (!on) return;
  const int qk = a->qk_bf16 ? 2 : (a->q_scale != nullptr ? 0 : 1);
  const int key = qk * 3 + a->pv_mode;  // pv_mode in 0..2 after validation
  static std::atomic<uint32_t> seen{0};
  if (seen.fetch_or(1u << key) & (1u << key)) return;
  static const char* const qk_name[] = {"MXFP8 (E4M3, E8M0 per 32 along head_dim)", "E4M3 per-tensor", "BF16"};
  static const char* const v_name[] = {"BF16 (P rounded to BF16)", "E4M3 unscaled, dequant scale 1.0 (P unscaled E4M3)",
                                       "MXFP8 along tokens (P unscaled E4M3)"};
  std::fprintf(stderr, "lpfa: lp_attn_varlen_fwd: Q/K %s, V %s, descales q/k/v %s/%s/%s\n", qk_name[qk],
               v_name[a->pv_mode], a->q_descale ? "yes" : "none", a->k_descale ? "yes" : "none",
               a->v_descale ? "yes" : "none");
}

}  // namespace

extern "C" {

int lpfa_abi_version(void) { return LPFA_ABI_VERSION; }

const char* lpfa_last_error(void) { return lpfa::last_error(); }

int mxfp8_quantize_varlen(const void* x, int x_dtype, int64_t stride_tok, int64_t stride_head,
                          int64_t total_tokens, int32_t num_heads, int32_t head_dim,
                          const int32_t* cu_seqlens, const int32_t* cu_scale, int32_t num_seqs,
                          int64_t total_scale_rows, int scaling_mode, uint8_t* payload,
                          uint8_t* scales, uint8_t* group_max, uint16_t* deq, void* stream) {
  if (int rc = lpfa::check_quantize(x, x_dtype, stride_tok, stride_head, total_tokens, num_heads,
                                    head_dim, cu_seqlens, cu_scale, num_seqs, total_scale_rows,
                                    scaling_mode, payload, scales))
    return rc;
  if (deq != nullptr && (reinterpret_cast<uintptr_t>(deq) & 15u)) {
    lpfa::set_error("deq is not 16-byte aligned");
    return LPFA_EINVAL;
  }
  lpfa::QuantParams p{};
  p.x = x;
  p.x_dtype = x_dtype;
  p.scaling_mode = scaling_mode;
  p.stride_tok = stride_tok;
  p.stride_head = stride_head;
  p.num_heads = num_heads;
  p.num_seqs = num_seqs;
  p.total_scale_rows = total_scale_rows;
  p.cu_seqlens = cu_seqlens;
  p.cu_scale = cu_scale;
  p.payload = payload;
  p.scales = scales;
  p.group_max = group_max;
  p.deq = deq;
  return launch_status(lpfa::launch_quantize(p, static_cast<hipStream_t>(stream)), "quantize");
}

int mxfp8_quantize_varlen_tokens(const void* x, int x_dtype, int64_t stride_tok, int64_t stride_head,
                                 int64_t total_tokens, int32_t num_heads, int32_t head_dim,
                                 const int32_t* cu_seqlens, const int32_t* cu_scale, int32_t num_seqs,
                                 int64_t total_scale_rows, int scaling_mode, uint8_t* payload,
                                 uint8_t* scales, void* stream) {
  if (int rc = lpfa::check_quantize(x, x_dtype, stride_tok, stride_head, total_tokens, num_heads,
                                    head_dim, cu_seqlens, cu_scale, num_seqs, total_scale_rows,
                                    scaling_mode, payload, scales))
    return rc;
  lpfa::QuantParams p{};
  p.x = x;
  p.x_dtype = x_dtype;
  p.scaling_mode = scaling_mode;
  p.stride_tok = stride_tok;
  p.stride_head = stride_head;
  p.num_heads = num_heads;
  p.num_seqs = num_seqs;
  p.total_scale_rows = total_scale_rows;
  p.cu_seqlens = cu_seqlens;
  p.cu_scale = cu_scale;
  p.payload = payload;
  p.scales = scales;
  return launch_status(lpfa::launch_quantize_tokens(p, static_cast<hipStream_t>(stream)), "token quantize");
}

int mxfp8_prepare_qkv(const void* q, const void* k, const void* v, int x_dtype, int64_t stride_tok,
                      int64_t stride_head, int64_t total_q, int64_t total_k, int32_t num_heads,
                      int32_t head_dim, const int32_t* cu_seqlens_q, const int32_t* cu_scale_q,
                      const int32_t* cu_seqlens_k, const int32_t* cu_scale_k, int32_t num_seqs,
                      int64_t total_scale_rows_q, int64_t total_scale_rows_k, int scaling_mode,
                      uint8_t* q_payload, uint8_t* q_scales, uint8_t* k_payload, uint8_t* k_scales,
                      uint8_t* k_group_max, uint8_t* v_codes, void* stream) {
  if (int rc = lpfa::check_quantize(q, x_dtype, stride_tok, stride_head, total_q, num_heads, head_dim,
                                    cu_seqlens_q, cu_scale_q, num_seqs, total_scale_rows_q, scaling_mode,
                                    q_payload, q_scales))
    return rc;
  if (int rc = lpfa::check_quantize(k, x_dtype, stride_tok, stride_head, total_k, num_heads, head_dim,
                                    cu_seqlens_k, cu_scale_k, num_seqs, total_scale_rows_k, scaling_mode,
                                    k_payload, k_scales))
    return rc;
  if (int rc = lpfa::check_cast(v, x_dtype, stride_tok, stride_head, total_k, num_heads, head_dim, v_codes))
    return rc;
  lpfa::QuantParams pq{}, pk{};
  for (lpfa::QuantParams* p : {&pq, &pk}) {
    p->x_dtype = x_dtype;
    p->scaling_mode = scaling_mode;
    p->stride_tok = stride_tok;
    p->stride_head = stride_head;
    p->num_heads = num_heads;
    p->num_seqs = num_seqs;
  }
  pq.x = q;
  pq.total_scale_rows = total_scale_rows_q;
  pq.cu_seqlens = cu_seqlens_q;
  pq.cu_scale = cu_scale_q;
  pq.payload = q_payload;
  pq.scales = q_scales;
  pk.x = k;
  pk.total_scale_rows = total_scale_rows_k;
  pk.cu_seqlens = cu_seqlens_k;
  pk.cu_scale = cu_scale_k;
  pk.payload = k_payload;
  pk.scales = k_scales;
  pk.group_max = k_group_max;
  lpfa::CastParams pv{};
  pv.x = v;
  pv.x_dtype = x_dtype;
  pv.stride_tok = stride_tok;
  pv.stride_head = stride_head;
  pv.total_tokens = total_k;
  pv.num_heads = num_heads;
  pv.y = v_codes;
  return launch_status(lpfa::launch_prepare_qkv(pq, pk, pv, static_cast<hipStream_t>(stream)), "prepare");
}

int lp_fp8_cast_e4m3(const void* x, int x_dtype, int64_t stride_tok, int64_t stride_head,
                     int64_t total_tokens, int32_t num_heads, int32_t head_dim, uint8_t* y,
                     uint8_t* group_max, void* stream) {
  if (int rc = lpfa::check_cast(x, x_dtype, stride_tok, stride_head, total_tokens, num_heads, head_dim, y))
    return rc;
  lpfa::CastParams p{};
  p.x = x;
  p.x_dtype = x_dtype;
  p.stride_tok = stride_tok;
  p.stride_head = stride_head;
  p.total_tokens = total_tokens;
  p.num_heads = num_heads;
  p.y = y;
  p.group_max = group_max;
  return launch_status(lpfa::launch_cast(p, static_cast<hipStream_t>(stream)), "e4m3 cast");
}

int lp_fp8_cast_current(const void* x, int x_dtype, int64_t stride_tok, int64_t stride_head,
                        int64_t total_tokens, int32_t num_heads, int32_t head_dim, float* work, uint8_t* y,
                        float* descale, void* stream) {
  if (int rc = lpfa::check_cast(x, x_dtype, stride_tok, stride_head, total_tokens, num_heads, head_dim, y))
    return rc;
  if (work == nullptr || descale == nullptr) {
    lpfa::set_error("work / descale is NULL");
    return LPFA_EINVAL;
  }
  if ((reinterpret_cast<uintptr_t>(work) & 3u) || (reinterpret_cast<uintptr_t>(descale) & 3u)) {
    lpfa::set_error("work / descale is not 4-byte aligned");
    return LPFA_EINVAL;
  }
  lpfa::CastParams p{};
  p.x = x;
  p.x_dtype = x_dtype;
  p.stride_tok = stride_tok;
  p.stride_head = stride_head;
  p.total_tokens = total_tokens;
  p.num_heads = num_heads;
  p.y = y;
  p.amax = work;
  p.descale = descale;
  return launch_status(lpfa::launch_cast_current(p, static_cast<hipStream_t>(stream)), "current-scaled cast");
}

int lp_fp8_cast_current_noalloc(const void* x, int x_dtype, int64_t stride_tok, int64_t stride_head,
                                int64_t total_tokens, int32_t num_heads, int32_t head_dim, uint8_t* y,
                                float* descale, void* stream) {
  if (int rc = lpfa::check_cast(x, x_dtype, stride_tok, stride_head, total_tokens, num_heads, head_dim, y))
    return rc;
  if (descale == nullptr || (reinterpret_cast<uintptr_t>(descale) & 3u)) {
    lpfa::set_error("descale is NULL or not 4-byte aligned");
    return LPFA_EINVAL;
  }
  float* ws = nullptr;
  int capacity = 0;
  if (hipError_t e = lpfa::current_scratch(&ws, &capacity); e != hipSuccess) {
    lpfa::set_error(std::string("static scratch address: ") + hipGetErrorString(e));
    return LPFA_EIO;
  }
  if (capacity < LPFA_CURRENT_WORK_FLOATS) {  // the partial maxima of any input size fit
    lpfa::set_error("static scratch smaller than the current-scaling workspace");
    return LPFA_EINVAL;
  }
  lpfa::CastParams p{};
  p.x = x;
  p.x_dtype = x_dtype;
  p.stride_tok = stride_tok;
  p.stride_head = stride_head;
  p.total_tokens = total_tokens;
  p.num_heads = num_heads;
  p.y = y;
  p.amax = ws;
  p.descale = descale;
  return launch_status(lpfa::launch_cast_current(p, static_cast<hipStream_t>(stream)), "current-scaled cast");
}

int lp_attn_varlen_fwd(const lpfa_attn_args* a, void* stream) {
  if (int rc = lpfa::check_attn(a)) return rc;
  log_variant_once(a);
  lpfa::AttnParams p{};
  p.q = a->q;
  p.k = a->k;
  p.v = a->v;
  p.q_scale = a->q_scale;
  p.k_scale = a->k_scale;
  p.cu_scale_q = a->cu_scale_q;
  p.cu_scale_k = a->cu_scale_k;
  p.cu_q = a->cu_seqlens_q;
  p.cu_k = a->cu_seqlens_k;
  p.q_descale = a->q_descale;
  p.k_descale = a->k_descale;
  p.v_descale = a->v_descale;
  p.tile_order = a->tile_order;
  p.out = a->out;
  p.lse = a->lse;
  p.q_st = a->q_stride_tok;
  p.q_sh = a->q_stride_head;
  p.k_st = a->k_stride_tok;
  p.k_sh = a->k_stride_head;
  p.v_st = a->v_stride_tok;
  p.v_sh = a->v_stride_head;
  p.qd_ss = a->q_descale_stride_seq;
  p.qd_sh = a->q_descale_stride_head;
  p.kd_ss = a->k_descale_stride_seq;
  p.kd_sh = a->k_descale_stride_head;
  p.vd_ss = a->v_descale_stride_seq;
  p.vd_sh = a->v_descale_stride_head;
  {
    // one past the last byte of the K and V tensors (the kernel's loads are range-checked)
    const int64_t vb = a->pv_mode == LPFA_PV_BF16 ? 2 : 1;
    const int64_t kb = a->qk_bf16 ? 2 : 1;
    const int64_t kspan = a->total_k > 0 ? ((a->total_k - 1) * a->k_stride_tok + (int64_t)(a->num_heads - 1) * a->k_stride_head + 128) * kb : 0;
    const int64_t vspan = a->total_k > 0 ? ((a->total_k - 1) * a->v_stride_tok + (int64_t)(a->num_heads - 1) * a->v_stride_head + 128) * vb : 0;
    p.k_end = a->k + kspan;
    p.k_gmax = a->qk_bf16 ? nullptr : a->k_scale_group_max;  // MX scale maxima or per-tensor code maxima
    p.v_scale = a->v_scale;
    p.qk_bf16 = a->qk_bf16;
    p.guard = a->fp8_score_guard == 0.0f ? LPFA_FP8_SCORE_GUARD_DEFAULT : a->fp8_score_guard;
    p.v_end = static_cast<const uint8_t*>(a->v) + vspan;
    p.k_deq = static_cast<const uint8_t*>(a->k_deq);
    p.k_deq_end = p.k_deq ? p.k_deq + a->total_k * a->num_heads * 256 : nullptr;
  }
  p.total_q = a->total_q;
  p.num_heads = a->num_heads;
  p.num_seqs = a->num_seqs;
  p.q_tiles = (a->max_seqlen_q + 127) / 128;
  p.num_tiles = a->tile_order ? a->num_tiles : a->num_seqs * a->num_heads * p.q_tiles;
  p.scale_log2 = a->softmax_scale * 1.4426950408889634f;
  return launch_status(lpfa::launch_attention(p, a->q_scale != nullptr, a->pv_mode, static_cast<hipStream_t>(stream),
                                               static_cast<hipEvent_t>(a->start_event),
                                               static_cast<hipEvent_t>(a->stop_event)),
                       "attention");
}

int lp_attn_varlen_bwd(const lpfa_bwd_args* a, void* stream) {
  if (int rc = lpfa::check_bwd(a)) return rc;
  lpfa::BwdParams p{};
  p.q = a->q;
  p.q_scale = a->q_scale;
  p.k = a->k;
  p.k_scale = a->k_scale;
  p.v = a->v;
  p.v_scale = a->v_scale;
  p.q_t = a->q_t;
  p.q_t_scale = a->q_t_scale;
  p.k_t = a->k_t;
  p.k_t_scale = a->k_t_scale;
  p.out = static_cast<const uint16_t*>(a->out);
  p.dout = static_cast<const uint16_t*>(a->dout);
  p.lse = a->lse;
  p.cu_q = a->cu_seqlens_q;
  p.cu_k = a->cu_seqlens_k;
  p.cu_scale_q = a->cu_scale_q;
  p.cu_scale_k = a->cu_scale_k;
  {
    // workspace: D, then BF16 copies of Qd, Qt, Kd, Vd, Kt (LPFA_BWD_WORK_BYTES)
    uint8_t* w = static_cast<uint8_t*>(a->work);
    const int64_t dbytes = ((int64_t)a->num_heads * a->total_q * 4 + 255) / 256 * 256;
    const int64_t qb = (int64_t)a->num_heads * 256 * a->total_q, kb = (int64_t)a->num_heads * 256 * a->total_k;
    p.delta = reinterpret_cast<float*>(w);
    p.qd16 = reinterpret_cast<uint16_t*>(w + dbytes);
    p.qt16 = reinterpret_cast<uint16_t*>(w + dbytes + qb);
    p.kd16 = reinterpret_cast<uint16_t*>(w + dbytes + 2 * qb);
    p.vd16 = reinterpret_cast<uint16_t*>(w + dbytes + 2 * qb + kb);
    p.kt16 = reinterpret_cast<uint16_t*>(w + dbytes + 2 * qb + 2 * kb);
  }
  p.dq = static_cast<uint16_t*>(a->dq);
  p.dk = static_cast<uint8_t*>(a->dk);
  p.dv = static_cast<uint8_t*>(a->dv);
  p.dk_scale = a->dk_scale;
  p.dv_scale = a->dv_scale;
  p.total_q = a->total_q;
  p.total_k = a->total_k;
  // with no keys (or no queries) there is nothing to contract: only the other side's zero or
  // pad outputs are written
  p.rows_q = a->total_q > 0 ? a->total_scale_rows_q : 0;
  p.rows_k = a->total_k > 0 ? a->total_scale_rows_k : 0;
  p.num_seqs = a->num_seqs;
  p.num_heads = a->num_heads;
  p.softmax_scale = a->softmax_scale;
  p.mx_dkv = a->output_mxfp8_dkv;
  p.scaling_mode = a->scaling_mode;
  return launch_status(lpfa::launch_attention_bwd(p, static_cast<hipStream_t>(stream)), "attention backward");
}

}  // extern "C"
