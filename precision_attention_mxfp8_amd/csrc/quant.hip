// MXFP8 quantizer and unscaled E4M3 cast for packed (tokens, heads, 128) tensors, gfx950.
//
// What is computed follows the LP-FA4 README (section "MXFP8 forward and backward"):
// E4M3 payload, one E8M0 scale per 32-element block along head_dim, per-sequence scale
// storage padded to 128 tokens, RCEIL default and FLOOR optional. The V cast follows the
// FastVideo fp8-PV PR (unscaled e4m3 cast of V).
//
// Work mapping (HBM-bound, one pass over the input):
//   A workgroup owns 16 consecutive rows of the scale storage for one head; 16 lanes own one
//   (scale row, head) pair = 128 elements; each lane loads 8
//   consecutive elements with one 16-byte load (two for FP32). The 4 lanes of a 32-element
//   block reduce their maximum with two cross-lane xor steps inside a quad (DPP), derive the
//   exponent from the maximum's bits, scale by an exact power of two and convert with the
//   hardware E4M3 conversion (round to nearest even). Lane 0 of the 16 gathers the four scale
//   bytes and writes them as one word. Pad rows of the scale storage get 0x7F and no payload.
//   Optionally the workgroup also writes the largest scale byte of its 16 rows' real rows (one
//   byte per 16-row group and head, 0 for a group of pad rows only): the attention kernel's
//   precision guard bounds |k| with it.
// The token-orientation quantizer (V for the P V product) takes blocks of 32 consecutive
// tokens of a sequence per (head, column); its mapping is described at the kernel.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_common.h"
#include "kernels.h"

namespace lpfa {

namespace {

template <typename T>
struct Loader;

template <>
struct Loader<uint16_t> {  // BF16 bit patterns: 8 elements = one 16-byte load
  __device__ static void load8(const void* base, int64_t off, float v[8]) {
    uint4 w = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(base) + off);
    uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = bf16_lo(u[i]);
      v[2 * i + 1] = bf16_hi(u[i]);
    }
  }
};

template <>
struct Loader<float> {  // FP32: 8 elements = two 16-byte loads
  __device__ static void load8(const void* base, int64_t off, float v[8]) {
    const float4* p = reinterpret_cast<const float4*>(reinterpret_cast<const float*>(base) + off);
    float4 a = p[0], b = p[1];
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
};

// One workgroup's share of the quantizer: 16 rows of the scale storage for one head (`bid`
// enumerates (16-row group, head) pairs, heads fastest).
template <typename T>
__device__ __forceinline__ void quantize_group(const QuantParams& p, unsigned bid, uint32_t* red) {
  const int h = (int)(bid % (unsigned)p.num_heads);  // neighbouring workgroups: same rows
  const int64_t grp16 = bid / (unsigned)p.num_heads;  // 16-row group of the scale storage
  const int sub = threadIdx.x & 15;                           // 8-element chunk of the 128-element row
  const int64_t srow = grp16 * 16 + (threadIdx.x >> 4);

  // sequence owning this group (groups never straddle sequences: each sequence's scale rows are
  // padded to a multiple of 128): the largest i with cu_scale[i] <= srow
  int lo = 0, hi = p.num_seqs;
  while (hi - lo > 1) {
    int mid = (lo + hi) >> 1;
    if ((int64_t)p.cu_scale[mid] <= srow) lo = mid; else hi = mid;
  }
  const int64_t local = srow - p.cu_scale[lo];
  const int64_t seq_len = (int64_t)p.cu_seqlens[lo + 1] - p.cu_seqlens[lo];
  uint32_t* scale_word = reinterpret_cast<uint32_t*>(p.scales + (srow * p.num_heads + h) * 4);
  uint32_t smax = 0;
  if (local >= seq_len) {  // pad row of the 128-token-padded scale storage
    if (sub == 0) *scale_word = 0x7F7F7F7Fu;
  } else {
    const int64_t t = p.cu_seqlens[lo] + local;
    float v[8];
    Loader<T>::load8(p.x, t * p.stride_tok + h * p.stride_head + sub * 8, v);
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
    // reduce over the 4 lanes of the 32-element block (lanes 4b..4b+3 of the 16)
    amax = fmaxf(amax, __shfl_xor(amax, 1));
    amax = fmaxf(amax, __shfl_xor(amax, 2));
    const int e = block_exponent(amax, p.scaling_mode);
    const float inv = __uint_as_float((uint32_t)(127 - e) << 23);  // 2^-e, e in [-127, 120]: normal

    uint32_t w0 = cvt4_e4m3(clamp448(v[0] * inv), clamp448(v[1] * inv), clamp448(v[2] * inv), clamp448(v[3] * inv));
    uint32_t w1 = cvt4_e4m3(clamp448(v[4] * inv), clamp448(v[5] * inv), clamp448(v[6] * inv), clamp448(v[7] * inv));
    *reinterpret_cast<uint2*>(p.payload + (t * p.num_heads + h) * 128 + sub * 8) = make_uint2(w0, w1);

    // gather the 4 block scale bytes of this row into lane 0 of the 16 (all 16 lanes of a row
    // take this branch together: the row decides it)
    const uint32_t sbyte = (uint32_t)(e + 127);
    smax = sbyte;
    const int base = (threadIdx.x & 63) & ~15;
    uint32_t b1 = __shfl(sbyte, base + 4);
    uint32_t b2 = __shfl(sbyte, base + 8);
    uint32_t b3 = __shfl(sbyte, base + 12);
    if (sub == 0) *scale_word = sbyte | (b1 << 8) | (b2 << 16) | (b3 << 24);
  }

  if (p.group_max != nullptr) {  // uniform over the workgroup
#pragma unroll
    for (int s = 1; s < 64; s <<= 1) smax = max(smax, (uint32_t)__shfl_xor((int)smax, s));
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = smax;
    __syncthreads();
    if (threadIdx.x == 0)
      p.group_max[grp16 * p.num_heads + h] = (uint8_t)max(max(red[0], red[1]), max(red[2], red[3]));
  }
}

template <typename T>
__global__ __launch_bounds__(256) void mxfp8_quantize_kernel(QuantParams p) {
  __shared__ uint32_t red[4];
  quantize_group<T>(p, blockIdx.x, red);
}

// Loads 4 consecutive elements (8 bytes BF16, 16 bytes FP32) as floats.
template <typename T>
__device__ __forceinline__ void load4(const void* base, int64_t off, float v[4]) {
  if constexpr (sizeof(T) == 2) {
    const uint2 w = *reinterpret_cast<const uint2*>(reinterpret_cast<const uint16_t*>(base) + off);
    v[0] = bf16_lo(w.x); v[1] = bf16_hi(w.x); v[2] = bf16_lo(w.y); v[3] = bf16_hi(w.y);
  } else {
    const float4 f = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(base) + off);
    v[0] = f.x; v[1] = f.y; v[2] = f.z; v[3] = f.w;
  }
}

// Token orientation: a workgroup owns one 32-token block (one row of the token-scale storage)
// of one head. Thread (token group tg = tid / 32, column group cg = tid % 32) holds tokens
// 4tg..4tg+3 and columns 4cg..4cg+3 (a wave reads two whole 256-byte BF16 rows per load).
// Column maxima: over the thread's 4 tokens, across the two token groups of a wave (lanes
// 32 apart), then across the 4 waves through LDS. Each thread then writes its 4x4 codes as
// four 4-byte words (a wave writes two whole 128-byte payload rows per store), and threads of
// token group 0 write the 128 scale bytes. Tokens past the sequence's end within its last
// block are neither read nor written; rows past its last block get 0x7F.
template <typename T>
__global__ __launch_bounds__(256) void mxfp8_quantize_tokens_kernel(QuantParams p) {
  __shared__ float red[4][128];
  const int h = (int)(blockIdx.x % (unsigned)p.num_heads);
  const int64_t brow = blockIdx.x / (unsigned)p.num_heads;  // row of the token-scale storage
  const int tid = threadIdx.x, cg = tid & 31, tg = tid >> 5, wv = tid >> 6;
  // owning sequence: the largest i with cu_scale[i] / 32 <= brow
  int lo = 0, hi = p.num_seqs;
  while (hi - lo > 1) {
    int mid = (lo + hi) >> 1;
    if ((int64_t)p.cu_scale[mid] / 32 <= brow) lo = mid; else hi = mid;
  }
  const int64_t blk = brow - (int64_t)p.cu_scale[lo] / 32;
  const int64_t len = (int64_t)p.cu_seqlens[lo + 1] - p.cu_seqlens[lo];
  uint32_t* scale_words = reinterpret_cast<uint32_t*>(p.scales + (brow * p.num_heads + h) * 128);
  if (32 * blk >= len) {  // past the sequence's last block (uniform over the workgroup)
    if (tg == 0) scale_words[cg] = 0x7F7F7F7Fu;
    return;
  }
  const int64_t t0 = p.cu_seqlens[lo] + 32 * blk;
  const int nval = (int)min<int64_t>(32, len - 32 * blk);  // real tokens in this block
  float v[4][4];
  float amax[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int tok = 4 * tg + r;
    const bool in = tok < nval;
    // a token past the end reads the block's first token (always real) and is then zeroed
    load4<T>(p.x, (t0 + (in ? tok : 0)) * p.stride_tok + h * p.stride_head + 4 * cg, v[r]);
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      if (!in) v[r][c] = 0.0f;
      amax[c] = fmaxf(amax[c], fabsf(v[r][c]));
    }
  }
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    amax[c] = fmaxf(amax[c], __shfl_xor(amax[c], 32));
    if ((tid & 63) < 32) red[wv][4 * cg + c] = amax[c];
  }
  __syncthreads();
  int e[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int col = 4 * cg + c;
    const float m = fmaxf(fmaxf(red[0][col], red[1][col]), fmaxf(red[2][col], red[3][col]));
    e[c] = block_exponent(m, p.scaling_mode);
  }
  if (tg == 0)
    scale_words[cg] = (uint32_t)(e[0] + 127) | ((uint32_t)(e[1] + 127) << 8) | ((uint32_t)(e[2] + 127) << 16) |
                      ((uint32_t)(e[3] + 127) << 24);
  float inv[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) inv[c] = __uint_as_float((uint32_t)(127 - e[c]) << 23);  // 2^-e, normal
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int tok = 4 * tg + r;
    if (tok < nval)
      *reinterpret_cast<uint32_t*>(p.payload + ((t0 + tok) * p.num_heads + h) * 128 + 4 * cg) =
          cvt4_e4m3(clamp448(v[r][0] * inv[0]), clamp448(v[r][1] * inv[1]), clamp448(v[r][2] * inv[2]),
                    clamp448(v[r][3] * inv[3]));
  }
}

template <typename T>
__device__ __forceinline__ void cast_block(const CastParams& p, unsigned bid) {
  const int64_t gid = (int64_t)bid * 256 + threadIdx.x;
  const int64_t head_row = gid >> 4;
  const int sub = threadIdx.x & 15;
  if (head_row >= p.total_tokens * p.num_heads) return;
  const int64_t t = head_row / p.num_heads;
  const int h = (int)(head_row - t * p.num_heads);
  float v[8];
  Loader<T>::load8(p.x, t * p.stride_tok + h * p.stride_head + sub * 8, v);
  uint32_t w0 = cvt4_e4m3(clamp448(v[0]), clamp448(v[1]), clamp448(v[2]), clamp448(v[3]));
  uint32_t w1 = cvt4_e4m3(clamp448(v[4]), clamp448(v[5]), clamp448(v[6]), clamp448(v[7]));
  *reinterpret_cast<uint2*>(p.y + head_row * 128 + sub * 8) = make_uint2(w0, w1);
}

template <typename T>
__global__ __launch_bounds__(256) void e4m3_cast_kernel(CastParams p) {
  cast_block<T>(p, blockIdx.x);
}

// The three preparation passes of a forward in one launch: Q's and K's MXFP8 quantization and
// V's unscaled E4M3 cast. Each of these passes moves ~12 MB at the dense shape, too little for
// one launch to get past its ramp-up and tail; one grid over all three amortizes them. Workgroup
// ranges: [0, nq) Q, [nq, nq + nk) K, then V; each workgroup runs one pass's body unchanged.
template <typename T>
__global__ __launch_bounds__(256) void prepare_qkv_kernel(QuantParams pq, QuantParams pk, CastParams pv, unsigned nq,
                                                          unsigned nk) {
  __shared__ uint32_t red[4];
  const unsigned b = blockIdx.x;
  if (b < nq) quantize_group<T>(pq, b, red);
  else if (b < nq + nk) quantize_group<T>(pk, b - nq, red);
  else cast_block<T>(pv, b - nq - nk);
}

// ---- per-tensor current scaling (TensorRT-LLM TE-backend PR: Q/K/V and O scales written from
// the current tensors before every call): amax over the whole tensor, then E4M3(x / s) with
// s = amax / 448 in float32 (1 for an all-zero tensor). Two kernels and no atomics: at most
// AMAX_BLOCKS workgroups each write the maximum of their share into work[1 + block], and every
// workgroup of the cast reduces those partial maxima before casting (work[0] receives amax).
constexpr int AMAX_BLOCKS = 256;

__device__ __forceinline__ int amax_blocks(int64_t chunks) {
  const int64_t b = (chunks + 255) / 256;
  return (int)(b < AMAX_BLOCKS ? b : AMAX_BLOCKS);
}

template <typename T>
__global__ __launch_bounds__(256) void amax_kernel(CastParams p) {
  __shared__ float red[4];
  const int64_t chunks = p.total_tokens * p.num_heads * 16;  // 8-element chunks
  const int64_t stride = (int64_t)gridDim.x * 256;
  float m = 0.0f;
  // a stride loop with 4 independent 16-byte loads in flight per thread
  for (int64_t c0 = (int64_t)blockIdx.x * 256 + threadIdx.x; c0 < chunks; c0 += 4 * stride) {
    float v[4][8];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      int64_t c = c0 + u * stride;
      c = c < chunks ? c : c0;  // a chunk past the end rereads this thread's first one (no effect on the max)
      const int64_t head_row = c >> 4;
      const int64_t t = head_row / p.num_heads;
      const int h = (int)(head_row - t * p.num_heads);
      Loader<T>::load8(p.x, t * p.stride_tok + h * p.stride_head + (c & 15) * 8, v[u]);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(v[u][i]));
  }
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) m = fmaxf(m, __shfl_xor(m, o));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) p.amax[1 + blockIdx.x] = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

template <typename T>
__global__ __launch_bounds__(256) void cast_current_kernel(CastParams p) {
  __shared__ float red[4];
  const int64_t chunks = p.total_tokens * p.num_heads * 16;
  const int nb = chunks > 0 ? amax_blocks(chunks) : 0;
  float m = (int)threadIdx.x < nb ? p.amax[1 + threadIdx.x] : 0.0f;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) m = fmaxf(m, __shfl_xor(m, o));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  const float amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float s = amax > 0.0f ? amax / 448.0f : 1.0f;  // IEEE division (round to nearest)
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (gid == 0) {
    p.amax[0] = amax;
    *p.descale = s;
  }
  const int64_t head_row = gid >> 4;
  if (head_row >= p.total_tokens * p.num_heads) return;
  const int64_t t = head_row / p.num_heads;
  const int h = (int)(head_row - t * p.num_heads);
  const int sub = threadIdx.x & 15;
  float v[8];
  Loader<T>::load8(p.x, t * p.stride_tok + h * p.stride_head + sub * 8, v);
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = clamp448(v[i] / s);  // the quotient rounded to float32 first
  const uint32_t w0 = cvt4_e4m3(v[0], v[1], v[2], v[3]), w1 = cvt4_e4m3(v[4], v[5], v[6], v[7]);
  *reinterpret_cast<uint2*>(p.y + head_row * 128 + sub * 8) = make_uint2(w0, w1);
}

}  // namespace

hipError_t launch_cast_current(const CastParams& p, hipStream_t s) {
  const int64_t chunks = p.total_tokens * p.num_heads * 16;
  const dim3 grid((unsigned)(chunks > 0 ? (chunks + 255) / 256 : 1));  // one block writes descale
  const dim3 agrid((unsigned)(grid.x < (unsigned)AMAX_BLOCKS ? grid.x : (unsigned)AMAX_BLOCKS));
  if (p.x_dtype == LPFA_DTYPE_BF16) {
    if (chunks > 0) hipLaunchKernelGGL(amax_kernel<uint16_t>, agrid, dim3(256), 0, s, p);
    hipLaunchKernelGGL(cast_current_kernel<uint16_t>, grid, dim3(256), 0, s, p);
  } else {
    if (chunks > 0) hipLaunchKernelGGL(amax_kernel<float>, agrid, dim3(256), 0, s, p);
    hipLaunchKernelGGL(cast_current_kernel<float>, grid, dim3(256), 0, s, p);
  }
  return hipGetLastError();
}

hipError_t launch_quantize(const QuantParams& p, hipStream_t s) {
  const int64_t groups = p.total_scale_rows / 16 * p.num_heads;  // scale rows: whole 128-row blocks
  if (groups == 0) return hipSuccess;
  const dim3 grid((unsigned)groups);
  if (p.x_dtype == LPFA_DTYPE_BF16)
    hipLaunchKernelGGL(mxfp8_quantize_kernel<uint16_t>, grid, dim3(256), 0, s, p);
  else
    hipLaunchKernelGGL(mxfp8_quantize_kernel<float>, grid, dim3(256), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_quantize_tokens(const QuantParams& p, hipStream_t s) {
  const int64_t blocks = p.total_scale_rows / 32 * p.num_heads;  // one per (32-token block, head)
  if (blocks == 0) return hipSuccess;
  const dim3 grid((unsigned)blocks);
  if (p.x_dtype == LPFA_DTYPE_BF16)
    hipLaunchKernelGGL(mxfp8_quantize_tokens_kernel<uint16_t>, grid, dim3(256), 0, s, p);
  else
    hipLaunchKernelGGL(mxfp8_quantize_tokens_kernel<float>, grid, dim3(256), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_prepare_qkv(const QuantParams& pq, const QuantParams& pk, const CastParams& pv, hipStream_t s) {
  const int64_t nq = pq.total_scale_rows / 16 * pq.num_heads, nk = pk.total_scale_rows / 16 * pk.num_heads;
  const int64_t nv = (pv.total_tokens * pv.num_heads * 16 + 255) / 256;
  if (nq + nk + nv == 0) return hipSuccess;
  const dim3 grid((unsigned)(nq + nk + nv));
  if (pq.x_dtype == LPFA_DTYPE_BF16)
    hipLaunchKernelGGL(prepare_qkv_kernel<uint16_t>, grid, dim3(256), 0, s, pq, pk, pv, (unsigned)nq, (unsigned)nk);
  else
    hipLaunchKernelGGL(prepare_qkv_kernel<float>, grid, dim3(256), 0, s, pq, pk, pv, (unsigned)nq, (unsigned)nk);
  return hipGetLastError();
}

hipError_t launch_cast(const CastParams& p, hipStream_t s) {
  const int64_t threads = p.total_tokens * p.num_heads * 16;
  if (threads == 0) return hipSuccess;
  const dim3 grid((unsigned)((threads + 255) / 256));
  if (p.x_dtype == LPFA_DTYPE_BF16)
    hipLaunchKernelGGL(e4m3_cast_kernel<uint16_t>, grid, dim3(256), 0, s, p);
  else
    hipLaunchKernelGGL(e4m3_cast_kernel<float>, grid, dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace lpfa
