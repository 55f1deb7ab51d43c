// Kernel parameter blocks and launchers (internal to the library).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "lpfa.h"

namespace lpfa {

struct QuantParams {
  const void* x;
  int x_dtype;
  int scaling_mode;
  int64_t stride_tok, stride_head;  // elements
  int32_t num_heads;
  int32_t num_seqs;
  int64_t total_scale_rows;
  const int32_t* cu_seqlens;
  const int32_t* cu_scale;
  uint8_t* payload;
  uint8_t* scales;
  uint8_t* group_max;  // optional: largest scale byte of each (16-row group, head)
  uint16_t* deq;       // optional: the quantized values as BF16, (T, H, 128) contiguous
};

struct CastParams {
  const void* x;
  int x_dtype;
  int64_t stride_tok, stride_head;
  int64_t total_tokens;
  int32_t num_heads;
  uint8_t* y;
  float* amax;     // current scaling: amax[0] = the tensor's largest magnitude; amax[1..256]: partial maxima
  float* descale;  // current scaling: s = amax / 448 (1 for an all-zero tensor)
  uint8_t* group_max;  // unscaled cast, optional: largest code magnitude of each (16 tokens, head)
};

struct AttnParams {
  const uint8_t* q;
  const uint8_t* k;
  const void* v;
  const uint8_t* q_scale;
  const uint8_t* k_scale;
  const int32_t* cu_scale_q;
  const int32_t* cu_scale_k;
  const int32_t* cu_q;
  const int32_t* cu_k;
  const float* q_descale;
  const float* k_descale;
  const float* v_descale;
  const int32_t* tile_order;
  uint16_t* out;
  float* lse;
  const uint8_t* k_gmax;   // optional K maxima per (16 rows, head): MX scale bytes / per-tensor code magnitudes
  const uint8_t* v_scale;  // V's token-block scales (MX V only)
  const uint8_t* k_end;    // one past the last byte of K / V: loads beyond read zeros
  const uint8_t* v_end;
  int64_t q_st, q_sh, k_st, k_sh, v_st, v_sh;  // elements
  int64_t qd_ss, qd_sh, kd_ss, kd_sh, vd_ss, vd_sh;
  int64_t total_q;
  int32_t num_heads;
  int32_t num_seqs;
  int32_t q_tiles;    // 128-query tiles per (sequence, head) in the default order
  int32_t num_tiles;  // work tiles to run
  float scale_log2;   // softmax_scale * log2(e)
  int32_t qk_bf16;    // Q and K are BF16 (the BF16 FlashAttention forward)
  float guard;        // FP8 scores when c * max|q| * max|k| <= guard (negative: never)
  const uint8_t* k_deq;      // optional: K's quantized values as BF16, (total_k, H, 128) contiguous
  const uint8_t* k_deq_end;  // one past its last byte
};

// Attention backward (lp_attn_varlen_bwd); every tensor contiguous, (tokens, heads, 128).
struct BwdParams {
  const uint8_t* q;
  const uint8_t* q_scale;
  const uint8_t* k;
  const uint8_t* k_scale;
  const uint8_t* v;
  const uint8_t* v_scale;
  const uint8_t* q_t;        // token orientation
  const uint8_t* q_t_scale;  // (scale rows / 32, H, 128)
  const uint8_t* k_t;
  const uint8_t* k_t_scale;
  const uint16_t* out;
  const uint16_t* dout;
  const float* lse;
  const int32_t* cu_q;
  const int32_t* cu_k;
  const int32_t* cu_scale_q;
  const int32_t* cu_scale_k;
  float* delta;  // -D = -rowsum(dO * O), (H, total_q), in the workspace
  // BF16 copies in the workspace (tokens, H, 128): Q and K in both orientations, V along head_dim
  uint16_t* qd16;
  uint16_t* qt16;
  uint16_t* kd16;
  uint16_t* vd16;
  uint16_t* kt16;
  uint16_t* dq;
  uint8_t* dk;   // BF16 bytes or E4M3 payload
  uint8_t* dv;
  uint8_t* dk_scale;
  uint8_t* dv_scale;
  int64_t total_q;
  int64_t total_k;
  int64_t rows_q;  // total scale rows of Q and K (multiples of 128)
  int64_t rows_k;
  int32_t num_seqs;
  int32_t num_heads;
  float softmax_scale;
  int32_t mx_dkv;
  int32_t scaling_mode;
};

hipError_t launch_quantize(const QuantParams& p, hipStream_t s);
hipError_t launch_quantize_tokens(const QuantParams& p, hipStream_t s);  // scales: token orientation
hipError_t launch_cast(const CastParams& p, hipStream_t s);
hipError_t launch_prepare_qkv(const QuantParams& pq, const QuantParams& pk, const CastParams& pv,
                              hipStream_t s);  // quantize Q, K and cast V in one launch (one dtype)
hipError_t launch_cast_current(const CastParams& p, hipStream_t s);  // amax, then E4M3(x / s)
// device address and size (floats) of the static scratch for current scaling on the current device
hipError_t current_scratch(float** out, int* capacity);
hipError_t launch_attention(const AttnParams& p, bool mx, int pv_mode, hipStream_t s,
                            hipEvent_t start = nullptr, hipEvent_t stop = nullptr);
hipError_t launch_attention_bwd(const BwdParams& p, hipStream_t s);  // D, then dK/dV, then dQ

}  // namespace lpfa
