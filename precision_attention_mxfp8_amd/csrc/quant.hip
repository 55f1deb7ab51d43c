// MXFP8 quantizer and unscaled E4M3 cast for packed (tokens, heads, 128) tensors, gfx950.
//
// What is computed follows the LP-FA4 README (section "MXFP8 forward and backward"):
// E4M3 payload, one E8M0 scale per 32-element block along head_dim, per-sequence scale
// storage padded to 128 tokens, RCEIL default and FLOOR optional. The V cast follows the
// FastVideo fp8-PV PR (unscaled e4m3 cast of V).
//
// Work mapping (HBM-bound, one pass over the input):
//   A workgroup is one wave and owns 16 consecutive rows of the scale storage for one head: a
//   16-lane row of the wave holds one (scale row, head) pair = 128 elements, 8 consecutive
//   elements per lane (one 16-byte load, two for FP32), and each lane takes four such rows, so
//   four loads per lane are in flight before any arithmetic. The 4 lanes of a 32-element block
//   reduce their maximum with two quad permutations (DPP), derive the exponent from the
//   maximum's bits and convert x * 2^-e to E4M3 with round to nearest even: BF16 input under
//   RCEIL with the scaled BF16 conversion straight from its bits, otherwise by multiplying with
//   an exact power of two and converting the product. Lane 0 of the 16 gathers the four scale
//   bytes with row shifts (DPP) and writes them as one word. Pad rows of the scale storage get
//   0x7F and no payload. Optionally the wave also writes the largest scale byte of its 16 rows' real rows
//   (one byte per 16-row group and head, 0 for a group of pad rows only): the attention
//   kernel's precision guard bounds |k| with it. Every cross-lane step stays inside a 16-lane
//   row, whose lanes are all real or all pad, except the four reads of the group maximum; no
//   step goes through LDS and no workgroup waits at a barrier.
// The token-orientation quantizer (V for the P V product) takes blocks of 32 consecutive
// tokens of a sequence per (head, column); its mapping is described at the kernel.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "device_common.h"
#include "kernels.h"

namespace lpfa {

namespace {

// An 8-element chunk as loaded (one 16-byte word for BF16, two for FP32), and its values. The
// quantizer and the cast by groups read their input once, with nontemporal loads: the input then
// does not displace from the L2 caches the codes these kernels write, which the attention reads
// next (one-launch preparation + attention at the dense shape: 35.56 -> 34.94 us per step; the
// preparation alone, replayed back to back, then reads its input from HBM: 5.8 -> 4.7 TB/s).
template <typename T>
__device__ __forceinline__ void load_chunk(const T* p, uint4 w[sizeof(T) / 2]) {
  typedef unsigned v4u_t __attribute__((ext_vector_type(4)));
#pragma unroll
  for (int k = 0; k < (int)sizeof(T) / 2; ++k) {
    const v4u_t x = __builtin_nontemporal_load(reinterpret_cast<const v4u_t*>(p) + k);
    w[k] = make_uint4(x.x, x.y, x.z, x.w);
  }
}
template <typename T>
__device__ __forceinline__ void unpack_chunk(const uint4 w[sizeof(T) / 2], float v[8]) {
  if constexpr (sizeof(T) == 2) {
    const uint32_t u[4] = {w[0].x, w[0].y, w[0].z, w[0].w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = bf16_lo(u[i]);
      v[2 * i + 1] = bf16_hi(u[i]);
    }
  } else {
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      v[4 * k] = __uint_as_float(w[k].x); v[4 * k + 1] = __uint_as_float(w[k].y);
      v[4 * k + 2] = __uint_as_float(w[k].z); v[4 * k + 3] = __uint_as_float(w[k].w);
    }
  }
}

// Cross-lane reads that stay inside 16-lane rows (DPP: no LDS round trip). dpp<CTRL>(x) returns
// the value x of the lane CTRL names, 0 where that lane lies outside the row.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)x, CTRL, 0xF, 0xF, true);
}
template <int CTRL>
__device__ __forceinline__ float dppf(float x) {
  return __uint_as_float(dpp<CTRL>(__float_as_uint(x)));
}
constexpr int QUAD_XOR1 = 0xB1;   // quad_perm [1,0,3,2]: lane i reads lane i ^ 1
constexpr int QUAD_XOR2 = 0x4E;   // quad_perm [2,3,0,1]: lane i reads lane i ^ 2
constexpr int ROW_SHL4 = 0x104;   // row_shl:n: lane i reads lane i + n of its row
constexpr int ROW_SHL8 = 0x108;
constexpr int ROW_SHL12 = 0x10C;
constexpr int ROW_ROR1 = 0x121;   // row_ror:n: lane i reads lane (i - n) mod 16 of its row
constexpr int ROW_ROR2 = 0x122;
constexpr int ROW_ROR4 = 0x124;
constexpr int ROW_ROR8 = 0x128;

constexpr int PREP_THREADS = 64;  // one wave per (16-row group, head)

// A read of the sequence offsets through the constant address space: they do not change while a
// kernel runs, and with a wave-uniform index this is a scalar load.
__device__ __forceinline__ int64_t ld_offset(const int32_t* p, int i) {
  return (int64_t)((const __attribute__((address_space(4))) int32_t*)(uintptr_t)p)[i];
}

// The largest of four lanes' values: lanes 0, 16, 32 and 48 (one per 16-lane row).
__device__ __forceinline__ uint32_t max_of_rows(uint32_t x) {
  const uint32_t a = (uint32_t)__builtin_amdgcn_readlane((int)x, 0), b = (uint32_t)__builtin_amdgcn_readlane((int)x, 16);
  const uint32_t c = (uint32_t)__builtin_amdgcn_readlane((int)x, 32), d = (uint32_t)__builtin_amdgcn_readlane((int)x, 48);
  return max(max(a, b), max(c, d));
}

// Four BF16 (two words) -> four E4M3 codes of x / 2^e in one word, first element in the low byte,
// with the hardware's scaled conversion; `scale` is 2^e built from the E8M0 byte (byte << 23, the
// zero pattern for e = -127). Checked on the GPU against the RNE conversion of x * 2^-e for every
// finite BF16 x and every e in [-127, 120] with |x| / 2^e <= 448: identical. Above 448 it gives NaN
// where the clamped path saturates, so only the RCEIL exponent (quotients <= 448) uses it.
__device__ __forceinline__ uint32_t cvt4_bf16_scaled(uint32_t w0, uint32_t w1, float scale) {
  typedef short v2s_t __attribute__((ext_vector_type(2)));
  typedef __bf16 v2bf_t __attribute__((ext_vector_type(2)));
  v2s_t r = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(v2s_t{0, 0}, __builtin_bit_cast(v2bf_t, w0), scale, false);
  r = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(r, __builtin_bit_cast(v2bf_t, w1), scale, true);
  return __builtin_bit_cast(uint32_t, r);
}

// The largest magnitude of eight BF16 (four words), as the float it stands for: magnitudes of
// finite BF16 order like their 15-bit patterns, so a packed 16-bit integer maximum finds it.
__device__ __forceinline__ float bf16x8_amax(uint4 w) {
  typedef unsigned short v2u16_t __attribute__((ext_vector_type(2)));
  const uint32_t M = 0x7FFF7FFFu;
  const v2u16_t a = __builtin_bit_cast(v2u16_t, w.x & M), b = __builtin_bit_cast(v2u16_t, w.y & M);
  const v2u16_t c = __builtin_bit_cast(v2u16_t, w.z & M), d = __builtin_bit_cast(v2u16_t, w.w & M);
  const v2u16_t m = __builtin_elementwise_max(__builtin_elementwise_max(a, b), __builtin_elementwise_max(c, d));
  return __uint_as_float(max((uint32_t)m[0], (uint32_t)m[1]) << 16);
}

// One wave's share of the quantizer: the 16 rows of the scale storage of one (16-row group,
// head). Lane l holds chunk l % 16 of the group's rows l / 16 + 4 i, i = 0..3. `real_rows` of the
// 16 rows are real (the rest are padding of the sequence's scale storage); FULL: all 16 are, so
// no per-row test is made. RCEIL: the exponent makes every |x| * 2^-e at most 448, so no clamp,
// and BF16 input converts with the scaled conversion straight from its bits (no unpacking and no
// multiplies). Per-wave bases are scalar and each lane's offsets are formed once.
template <typename T, bool RCEIL, bool FULL>
__device__ __forceinline__ void quantize_rows(const QuantParams& p, int h, int64_t grp16, int64_t first, int64_t local0,
                                              int real_rows) {
  const int64_t H = p.num_heads;
  const int lane = threadIdx.x, sub = lane & 15, q = lane >> 4;
  const int64_t row0 = grp16 * 16, tok0 = first + local0;  // tok0: the token of row0 (when it is real)

  // All four loads first. A pad row reads a real row of its sequence instead (the sequence has
  // at least one token, as it owns scale rows); a pad row's values reach no output, since every
  // cross-lane step of a row stays inside the row.
  constexpr int NW = sizeof(T) / 2;  // 16-byte words per 8-element chunk
  uint4 raw[4][NW];
  if constexpr (FULL) {
    const T* x0 = static_cast<const T*>(p.x) + tok0 * p.stride_tok + h * p.stride_head;
    const int64_t off = q * p.stride_tok + sub * 8;
#pragma unroll
    for (int i = 0; i < 4; ++i) load_chunk<T>(x0 + 4 * i * p.stride_tok + off, raw[i]);
  } else {
    const T* x0 = static_cast<const T*>(p.x) + (real_rows > 0 ? tok0 : first) * p.stride_tok + h * p.stride_head;
    const int last = real_rows > 0 ? real_rows - 1 : 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) load_chunk<T>(x0 + (int64_t)min(q + 4 * i, last) * p.stride_tok + sub * 8, raw[i]);
  }
  constexpr bool SCALED_CVT = RCEIL && sizeof(T) == 2;

  uint8_t* pay = p.payload + (tok0 * H + h) * 128 + (q * H * 128 + sub * 8);
  uint8_t* scw = p.scales + (row0 * H + h) * 4 + q * H * 4;
  uint32_t smax = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float v[8];
    float amax = 0.0f;
    if constexpr (SCALED_CVT) {
      amax = bf16x8_amax(raw[i][0]);
    } else {
      unpack_chunk<T>(raw[i], v);
#pragma unroll
      for (int j = 0; j < 8; ++j) amax = fmaxf(amax, fabsf(v[j]));
    }
    // the maximum over the 4 lanes of the 32-element block (lanes 4b..4b+3 of the row)
    amax = fmaxf(amax, dppf<QUAD_XOR1>(amax));
    amax = fmaxf(amax, dppf<QUAD_XOR2>(amax));
    const int e = block_exponent(amax, RCEIL ? LPFA_SCALING_RCEIL : LPFA_SCALING_FLOOR);
    const float inv = __uint_as_float((uint32_t)(127 - e) << 23);  // 2^-e, e in [-127, 120]: normal
    const uint32_t sbyte = (uint32_t)(e + 127);
    // the row's four block scales (lanes 0, 4, 8, 12), gathered into lane 0 of the row
    const uint32_t word = sbyte | (dpp<ROW_SHL4>(sbyte) << 8) | (dpp<ROW_SHL8>(sbyte) << 16) | (dpp<ROW_SHL12>(sbyte) << 24);
    uint32_t* scale_word = reinterpret_cast<uint32_t*>(scw + 4 * i * H * 4);
    if (FULL || q + 4 * i < real_rows) {
      uint32_t w0, w1;
      if constexpr (SCALED_CVT) {
        const float sc = __uint_as_float(sbyte << 23);  // 2^e
        w0 = cvt4_bf16_scaled(raw[i][0].x, raw[i][0].y, sc);
        w1 = cvt4_bf16_scaled(raw[i][0].z, raw[i][0].w, sc);
      } else {
        float y[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) y[j] = RCEIL ? v[j] * inv : clamp448(v[j] * inv);
        w0 = cvt4_e4m3(y[0], y[1], y[2], y[3]);
        w1 = cvt4_e4m3(y[4], y[5], y[6], y[7]);
      }
      *reinterpret_cast<uint2*>(pay + 4 * i * H * 128) = make_uint2(w0, w1);
      if (p.deq != nullptr) {  // uniform: the quantized values themselves, as BF16
        const float sc = __uint_as_float(sbyte << 23);
        const uint2 a = fp8x4_scaled_bf16(w0, sc), b = fp8x4_scaled_bf16(w1, sc);
        *reinterpret_cast<uint4*>(p.deq + (tok0 * H + h) * 128 + (q * H * 128 + sub * 8) + 4 * i * H * 128) =
            make_uint4(a.x, a.y, b.x, b.y);
      }
      if (sub == 0) *scale_word = word;
      smax = max(smax, sbyte);
    } else if (sub == 0) {
      *scale_word = 0x7F7F7F7Fu;  // pad row of the 128-row-padded scale storage
    }
  }

  if (p.group_max != nullptr) {  // uniform over the wave
    // each row's largest (over its lanes 0, 4, 8, 12 and, per lane, over its four rows), then the wave's
    smax = max(smax, dpp<ROW_ROR4>(smax));
    smax = max(smax, dpp<ROW_ROR8>(smax));
    const uint32_t g = max_of_rows(smax);
    if (lane == 0) p.group_max[grp16 * H + h] = (uint8_t)g;
  }
}

// One wave's share of the quantizer: the 16 rows of the scale storage of one (16-row group,
// head) (`bid` enumerates those pairs, heads fastest).
template <typename T>
__device__ __forceinline__ void quantize_group(const QuantParams& p, unsigned bid) {
  const int h = (int)(bid % (unsigned)p.num_heads);  // neighbouring workgroups: same rows
  const int64_t grp16 = bid / (unsigned)p.num_heads;  // 16-row group of the scale storage
  const int64_t row0 = grp16 * 16;
  // The sequence owning the group, the same for all its rows (every sequence's scale rows are
  // padded to a multiple of 128, so no group straddles two): the largest i with cu_scale[i] <=
  // row0. Uniform over the wave, so these reads are scalar loads.
  int lo = 0, hi = p.num_seqs;
  while (hi - lo > 1) {
    int mid = (lo + hi) >> 1;
    if (ld_offset(p.cu_scale, mid) <= row0) lo = mid; else hi = mid;
  }
  const int64_t local0 = row0 - ld_offset(p.cu_scale, lo);  // the group's first row within its sequence
  const int64_t first = ld_offset(p.cu_seqlens, lo);
  const int64_t left = ld_offset(p.cu_seqlens, lo + 1) - first - local0;  // real rows from row0 on
  const int real_rows = left <= 0 ? 0 : (left >= 16 ? 16 : (int)left);
  const bool rceil = p.scaling_mode == LPFA_SCALING_RCEIL;
  if (real_rows == 16) {
    if (rceil) quantize_rows<T, true, true>(p, h, grp16, first, local0, 16);
    else quantize_rows<T, false, true>(p, h, grp16, first, local0, 16);
  } else {
    if (rceil) quantize_rows<T, true, false>(p, h, grp16, first, local0, real_rows);
    else quantize_rows<T, false, false>(p, h, grp16, first, local0, real_rows);
  }
}

template <typename T>
__global__ __launch_bounds__(PREP_THREADS) void mxfp8_quantize_kernel(QuantParams p) {
  quantize_group<T>(p, blockIdx.x);
}

// Token orientation: a workgroup is one wave and owns one 32-token block (one row of the
// token-scale storage) of one head. Lane l holds the 8-column chunk l % 16 of tokens l / 16 + 4 i
// (i = 0..7), and its eight 16-byte loads (sixteen for FP32) go out first. Column maxima: over
// the lane's 8 tokens, then across the wave's four 16-lane rows (two shuffles per column, issued
// together). The lanes of the first row write the 128 scale bytes (8 each); every lane writes
// the 8 codes of each of its real tokens. Tokens past the sequence's end within its last block
// read the block's first token, count as zero and are not written; rows past its last block get
// 0x7F.
template <typename T>
__global__ __launch_bounds__(PREP_THREADS) void mxfp8_quantize_tokens_kernel(QuantParams p) {
  const int64_t H = p.num_heads;
  const int h = (int)(blockIdx.x % (unsigned)p.num_heads);
  const int64_t brow = blockIdx.x / (unsigned)p.num_heads;  // row of the token-scale storage
  const int lane = threadIdx.x, c = lane & 15, q = lane >> 4;
  // owning sequence (uniform: scalar loads): the largest i with cu_scale[i] / 32 <= brow
  int lo = 0, hi = p.num_seqs;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (ld_offset(p.cu_scale, mid) / 32 <= brow) lo = mid; else hi = mid;
  }
  const int64_t blk = brow - ld_offset(p.cu_scale, lo) / 32;
  const int64_t first = ld_offset(p.cu_seqlens, lo);
  const int64_t len = ld_offset(p.cu_seqlens, lo + 1) - first;
  uint2* scale_out = reinterpret_cast<uint2*>(p.scales + (brow * H + h) * 128 + 8 * c);
  if (32 * blk >= len) {  // past the sequence's last block (uniform over the wave)
    if (q == 0) *scale_out = make_uint2(0x7F7F7F7Fu, 0x7F7F7F7Fu);
    return;
  }
  const int64_t t0 = first + 32 * blk;
  const int n = (int)min<int64_t>(32, len - 32 * blk);  // real tokens in this block (>= 1)
  const T* x0 = static_cast<const T*>(p.x) + t0 * p.stride_tok + h * p.stride_head + 8 * c;
  uint4 raw[8][sizeof(T) / 2];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int tok = q + 4 * i;
    load_chunk<T>(x0 + (int64_t)(tok < n ? tok : 0) * p.stride_tok, raw[i]);
  }
  float cm[8] = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    if (q + 4 * i >= n) continue;
    float v[8];
    unpack_chunk<T>(raw[i], v);
#pragma unroll
    for (int j = 0; j < 8; ++j) cm[j] = fmaxf(cm[j], fabsf(v[j]));
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) cm[j] = fmaxf(cm[j], __shfl_xor(cm[j], 16));
#pragma unroll
  for (int j = 0; j < 8; ++j) cm[j] = fmaxf(cm[j], __shfl_xor(cm[j], 32));
  float inv[8];
  uint32_t sb[2] = {0u, 0u};
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int e = block_exponent(cm[j], p.scaling_mode);
    inv[j] = __uint_as_float((uint32_t)(127 - e) << 23);  // 2^-e, normal
    sb[j >> 2] |= (uint32_t)(e + 127) << (8 * (j & 3));
  }
  if (q == 0) *scale_out = make_uint2(sb[0], sb[1]);
  uint8_t* pay = p.payload + (t0 * H + h) * 128 + 8 * c;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int tok = q + 4 * i;
    if (tok >= n) continue;
    float v[8];
    unpack_chunk<T>(raw[i], v);
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = clamp448(v[j] * inv[j]);  // a no-op under RCEIL (|v| * 2^-e <= 448)
    *reinterpret_cast<uint2*>(pay + (int64_t)tok * H * 128) =
        make_uint2(cvt4_e4m3(v[0], v[1], v[2], v[3]), cvt4_e4m3(v[4], v[5], v[6], v[7]));
  }
}

// The cast by (16-token group, head): a workgroup is one wave and owns 16 consecutive tokens of
// one head (bid enumerates (16-token group, head), heads fastest, as the quantizer's groups do),
// laid out like the quantizer's rows: lane l holds chunk l % 16 of tokens l / 16 + 4 i. With group
// maxima (per-tensor K for the attention's precision guard) it also writes the largest code
// magnitude of its 2048 codes (codes order like magnitudes, and the RNE conversion is monotonic,
// so that is the code of the largest clamped magnitude). A token past the end reads the group's
// last real token instead and reaches no output. FULL: all 16 tokens are real; GMAX: the group
// maxima are written (p.group_max is set).
template <typename T, bool FULL, bool GMAX>
__device__ __forceinline__ void cast_rows(const CastParams& p, int h, int64_t g16) {
  const int64_t H = p.num_heads, t0 = g16 * 16;
  const int lane = threadIdx.x, sub = lane & 15, q = lane >> 4;
  // all four loads first; a token past the end reads the group's last real token instead
  const int n = FULL ? 16 : (int)(p.total_tokens - t0);  // real tokens in the group (>= 1)
  const T* x0 = static_cast<const T*>(p.x) + t0 * p.stride_tok + h * p.stride_head;
  uint4 raw[4][sizeof(T) / 2];
  if constexpr (FULL) {
    const int64_t off = q * p.stride_tok + sub * 8;
#pragma unroll
    for (int i = 0; i < 4; ++i) load_chunk<T>(x0 + 4 * i * p.stride_tok + off, raw[i]);
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) load_chunk<T>(x0 + (int64_t)min(q + 4 * i, n - 1) * p.stride_tok + sub * 8, raw[i]);
  }
  float v[4][8];
#pragma unroll
  for (int i = 0; i < 4; ++i) unpack_chunk<T>(raw[i], v[i]);
  uint8_t* y = p.y + (t0 * H + h) * 128 + (q * H * 128 + sub * 8);
  float m = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float mi = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      v[i][j] = clamp448(v[i][j]);
      if (GMAX) mi = fmaxf(mi, fabsf(v[i][j]));
    }
    if (FULL || q + 4 * i < n) {
      if (GMAX) m = fmaxf(m, mi);
      const uint32_t w0 = cvt4_e4m3(v[i][0], v[i][1], v[i][2], v[i][3]), w1 = cvt4_e4m3(v[i][4], v[i][5], v[i][6], v[i][7]);
      *reinterpret_cast<uint2*>(y + 4 * i * H * 128) = make_uint2(w0, w1);
    }
  }
  if (!GMAX) return;
  // the row's largest (rotations by 1, 2, 4 and 8 reach all 16 lanes), then the wave's
  m = fmaxf(m, dppf<ROW_ROR1>(m));
  m = fmaxf(m, dppf<ROW_ROR2>(m));
  m = fmaxf(m, dppf<ROW_ROR4>(m));
  m = fmaxf(m, dppf<ROW_ROR8>(m));
  const float g = __uint_as_float(max_of_rows(__float_as_uint(m)));  // non-negative: ordered like its bits
  if (lane == 0) p.group_max[g16 * H + h] = (uint8_t)(cvt_pk_e4m3(g, 0.0f) & 0x7Fu);
}

template <typename T>
__device__ __forceinline__ void cast_group(const CastParams& p, unsigned bid) {
  const int h = (int)(bid % (unsigned)p.num_heads);
  const int64_t g16 = bid / (unsigned)p.num_heads;
  const bool full = g16 * 16 + 16 <= p.total_tokens;
  if (p.group_max != nullptr) {
    if (full) cast_rows<T, true, true>(p, h, g16);
    else cast_rows<T, false, true>(p, h, g16);
  } else {
    if (full) cast_rows<T, true, false>(p, h, g16);
    else cast_rows<T, false, false>(p, h, g16);
  }
}

template <typename T>
__global__ __launch_bounds__(PREP_THREADS) void e4m3_cast_kernel(CastParams p) {
  cast_group<T>(p, blockIdx.x);
}

// The three preparation passes of a forward in one launch: Q's and K's MXFP8 quantization and
// V's unscaled E4M3 cast. Each of these passes moves ~12 MB at the dense shape, too little for
// one launch to get past its ramp-up and tail; one grid over all three amortizes them. Workgroup
// ranges: [0, nq) Q, [nq, nq + nk) K, then V; each workgroup runs one pass's body unchanged.
// V takes the (16-token group, head) mapping of the quantizer's groups, so with a head count that
// is a multiple of 8 every head's Q, K and V codes are written by workgroups of one XCD (ids are
// dealt round-robin over the 8 XCDs), the XCD whose L2 the attention kernel reads that head from.
template <typename T>
__global__ __launch_bounds__(PREP_THREADS) void prepare_qkv_kernel(QuantParams pq, QuantParams pk, CastParams pv,
                                                                   unsigned nq, unsigned nk) {
  const unsigned b = blockIdx.x;
  if (b < nq) quantize_group<T>(pq, b);
  else if (b < nq + nk) quantize_group<T>(pk, b - nq);
  else cast_group<T>(pv, b - nq - nk);
}

// ---- per-tensor current scaling (TensorRT-LLM TE-backend PR: Q/K/V and O scales written from
// the current tensors before every call): amax over the whole tensor, then E4M3(x / s) with
// s = amax / 448 in float32 (1 for an all-zero tensor). Two kernels and no atomics: at most
// AMAX_BLOCKS workgroups each write the maximum of their share into work[1 + block], and every
// workgroup of the cast reduces those partial maxima before casting (work[0] receives amax).
constexpr int AMAX_BLOCKS = 256;

__host__ __device__ __forceinline__ int amax_blocks(int64_t chunks) {
  const int64_t b = (chunks + 255) / 256;
  return (int)(b < AMAX_BLOCKS ? b : AMAX_BLOCKS);
}

template <typename T>
__global__ __launch_bounds__(256) void amax_kernel(CastParams p) {
  __shared__ float red[4];
  const int64_t chunks = p.total_tokens * p.num_heads * 16;  // 8-element chunks
  const int64_t stride = (int64_t)gridDim.x * 256;
  constexpr int U = 8;  // independent 16-byte loads in flight per thread (FP32: 16)
  // a packed tensor (heads and tokens back to back) is one run of chunks: no index arithmetic
  const bool packed = p.stride_head == 128 && p.stride_tok == (int64_t)p.num_heads * 128;
  float m = 0.0f;
  for (int64_t c0 = (int64_t)blockIdx.x * 256 + threadIdx.x; c0 < chunks; c0 += U * stride) {
    uint4 raw[U][sizeof(T) / 2];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      int64_t c = c0 + u * stride;
      c = c < chunks ? c : c0;  // a chunk past the end rereads this thread's first one (no effect on the max)
      int64_t off = c * 8;
      if (!packed) {
        const int64_t head_row = c >> 4;
        const int64_t t = head_row / p.num_heads;
        const int h = (int)(head_row - t * p.num_heads);
        off = t * p.stride_tok + h * p.stride_head + (c & 15) * 8;
      }
#pragma unroll
      for (int k = 0; k < (int)sizeof(T) / 2; ++k) raw[u][k] = reinterpret_cast<const uint4*>(static_cast<const T*>(p.x) + off)[k];
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float v[8];
      unpack_chunk<T>(raw[u], v);
#pragma unroll
      for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(v[i]));
    }
  }
  m = fmaxf(m, dppf<ROW_ROR1>(m));
  m = fmaxf(m, dppf<ROW_ROR2>(m));
  m = fmaxf(m, dppf<ROW_ROR4>(m));
  m = fmaxf(m, dppf<ROW_ROR8>(m));
  m = __uint_as_float(max_of_rows(__float_as_uint(m)));  // non-negative: ordered like its bits
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) p.amax[1 + blockIdx.x] = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

// The scaled cast by (16-token group, head), one wave each, laid out like the cast by groups: lane
// l holds chunk l % 16 of tokens l / 16 + 4 i. The wave's loads go out first; it then reduces the
// partial maxima itself (four per lane, DPP within rows, one read per row), so no workgroup waits
// at a barrier before its loads.
template <typename T, bool FULL>
__device__ __forceinline__ void cast_current_rows(const CastParams& p, int h, int64_t g16, int nb) {
  const int64_t H = p.num_heads, t0 = g16 * 16;
  const int lane = threadIdx.x, sub = lane & 15, q = lane >> 4;
  const int n = FULL ? 16 : (int)(p.total_tokens - t0);  // real tokens in the group (>= 1)
  const T* x0 = static_cast<const T*>(p.x) + t0 * p.stride_tok + h * p.stride_head;
  uint4 raw[4][sizeof(T) / 2];
  if constexpr (FULL) {
    const int64_t off = q * p.stride_tok + sub * 8;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int k = 0; k < (int)sizeof(T) / 2; ++k)
        raw[i][k] = reinterpret_cast<const uint4*>(x0 + 4 * i * p.stride_tok + off)[k];
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int k = 0; k < (int)sizeof(T) / 2; ++k)
        raw[i][k] = reinterpret_cast<const uint4*>(x0 + (int64_t)min(q + 4 * i, n - 1) * p.stride_tok + sub * 8)[k];
  }
  // amax over the partial maxima (at most 256: four per lane)
  float m = 0.0f;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int b = 4 * lane + j;
    if (b < nb) m = fmaxf(m, p.amax[1 + b]);
  }
  m = fmaxf(m, dppf<ROW_ROR1>(m));
  m = fmaxf(m, dppf<ROW_ROR2>(m));
  m = fmaxf(m, dppf<ROW_ROR4>(m));
  m = fmaxf(m, dppf<ROW_ROR8>(m));
  const float amax = __uint_as_float(max_of_rows(__float_as_uint(m)));
  const float s = amax > 0.0f ? amax / 448.0f : 1.0f;  // IEEE division (round to nearest)
  if (g16 == 0 && h == 0 && lane == 0) {
    p.amax[0] = amax;
    *p.descale = s;
  }
  uint8_t* y = p.y + (t0 * H + h) * 128 + (q * H * 128 + sub * 8);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (!FULL && q + 4 * i >= n) continue;
    float v[8];
    unpack_chunk<T>(raw[i], v);
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = clamp448(v[j] / s);  // the quotient rounded to float32 first
    const uint32_t w0 = cvt4_e4m3(v[0], v[1], v[2], v[3]), w1 = cvt4_e4m3(v[4], v[5], v[6], v[7]);
    *reinterpret_cast<uint2*>(y + 4 * i * H * 128) = make_uint2(w0, w1);
  }
}

template <typename T>
__global__ __launch_bounds__(PREP_THREADS) void cast_current_kernel(CastParams p) {
  const int64_t chunks = p.total_tokens * p.num_heads * 16;
  const int nb = chunks > 0 ? amax_blocks(chunks) : 0;
  if (chunks == 0) {  // an empty tensor: amax 0, descale 1
    if (threadIdx.x == 0) {
      p.amax[0] = 0.0f;
      *p.descale = 1.0f;
    }
    return;
  }
  const int h = (int)(blockIdx.x % (unsigned)p.num_heads);
  const int64_t g16 = blockIdx.x / (unsigned)p.num_heads;
  if (g16 * 16 + 16 <= p.total_tokens) cast_current_rows<T, true>(p, h, g16, nb);
  else cast_current_rows<T, false>(p, h, g16, nb);
}

// Scratch of the allocation-free current-scaling entry point: the partial maxima that
// amax_kernel hands to cast_current_kernel, in a file-scope device array instead of a caller
// workspace. Every GPU the library runs on holds its own copy (2 KB) until the process ends.
// Each call's amax_kernel writes all the partial maxima its cast_current_kernel reads, so nothing
// needs clearing; calls that overlap on one GPU share the array and race.
constexpr int CURRENT_SCRATCH_FLOATS = 512;
static_assert(CURRENT_SCRATCH_FLOATS >= 1 + AMAX_BLOCKS && LPFA_CURRENT_WORK_FLOATS == 1 + AMAX_BLOCKS,
              "scratch holds amax and every partial maximum");
static __device__ __align__(256) float scratch[CURRENT_SCRATCH_FLOATS];

}  // namespace

// The scratch array's device address on the current device. The name `scratch` in host code is a
// host-side stand-in, not a device address, so the address is looked up once per device and kept.
hipError_t current_scratch(float** out, int* capacity) {
  static std::mutex mu;
  static float* ptrs[64] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (ptrs[dev] == nullptr) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    ptrs[dev] = static_cast<float*>(ptr);
  }
  *out = ptrs[dev];
  *capacity = CURRENT_SCRATCH_FLOATS;
  return hipSuccess;
}

hipError_t launch_cast_current(const CastParams& p, hipStream_t s) {
  const int64_t chunks = p.total_tokens * p.num_heads * 16;
  // the cast: one wave per (16-token group, head); an empty tensor still gets one (it writes the
  // descale)
  const dim3 grid((unsigned)(chunks > 0 ? (p.total_tokens + 15) / 16 * p.num_heads : 1));
  const dim3 agrid((unsigned)(chunks > 0 ? amax_blocks(chunks) : 0));
  if (p.x_dtype == LPFA_DTYPE_BF16) {
    if (chunks > 0) hipLaunchKernelGGL(amax_kernel<uint16_t>, agrid, dim3(256), 0, s, p);
    hipLaunchKernelGGL(cast_current_kernel<uint16_t>, grid, dim3(PREP_THREADS), 0, s, p);
  } else {
    if (chunks > 0) hipLaunchKernelGGL(amax_kernel<float>, agrid, dim3(256), 0, s, p);
    hipLaunchKernelGGL(cast_current_kernel<float>, grid, dim3(PREP_THREADS), 0, s, p);
  }
  return hipGetLastError();
}

hipError_t launch_quantize(const QuantParams& p, hipStream_t s) {
  const int64_t groups = p.total_scale_rows / 16 * p.num_heads;  // scale rows: whole 128-row blocks
  if (groups == 0) return hipSuccess;
  const dim3 grid((unsigned)groups);
  if (p.x_dtype == LPFA_DTYPE_BF16)
    hipLaunchKernelGGL(mxfp8_quantize_kernel<uint16_t>, grid, dim3(PREP_THREADS), 0, s, p);
  else
    hipLaunchKernelGGL(mxfp8_quantize_kernel<float>, grid, dim3(PREP_THREADS), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_quantize_tokens(const QuantParams& p, hipStream_t s) {
  const int64_t blocks = p.total_scale_rows / 32 * p.num_heads;  // one per (32-token block, head)
  if (blocks == 0) return hipSuccess;
  const dim3 grid((unsigned)blocks);
  if (p.x_dtype == LPFA_DTYPE_BF16)
    hipLaunchKernelGGL(mxfp8_quantize_tokens_kernel<uint16_t>, grid, dim3(PREP_THREADS), 0, s, p);
  else
    hipLaunchKernelGGL(mxfp8_quantize_tokens_kernel<float>, grid, dim3(PREP_THREADS), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_prepare_qkv(const QuantParams& pq, const QuantParams& pk, const CastParams& pv, hipStream_t s) {
  const int64_t nq = pq.total_scale_rows / 16 * pq.num_heads, nk = pk.total_scale_rows / 16 * pk.num_heads;
  const int64_t nv = (pv.total_tokens + 15) / 16 * pv.num_heads;  // (16-token group, head) workgroups
  if (nq + nk + nv == 0) return hipSuccess;
  const dim3 grid((unsigned)(nq + nk + nv));
  if (pq.x_dtype == LPFA_DTYPE_BF16)
    hipLaunchKernelGGL(prepare_qkv_kernel<uint16_t>, grid, dim3(PREP_THREADS), 0, s, pq, pk, pv, (unsigned)nq, (unsigned)nk);
  else
    hipLaunchKernelGGL(prepare_qkv_kernel<float>, grid, dim3(PREP_THREADS), 0, s, pq, pk, pv, (unsigned)nq, (unsigned)nk);
  return hipGetLastError();
}

hipError_t launch_cast(const CastParams& p, hipStream_t s) {
  if (p.total_tokens * p.num_heads == 0) return hipSuccess;
  // one wave per (16-token group, head), with or without group maxima
  const dim3 grid((unsigned)((p.total_tokens + 15) / 16 * p.num_heads));
  if (p.x_dtype == LPFA_DTYPE_BF16)
    hipLaunchKernelGGL(e4m3_cast_kernel<uint16_t>, grid, dim3(PREP_THREADS), 0, s, p);
  else
    hipLaunchKernelGGL(e4m3_cast_kernel<float>, grid, dim3(PREP_THREADS), 0, s, p);
  return hipGetLastError();
}

}  // namespace lpfa
