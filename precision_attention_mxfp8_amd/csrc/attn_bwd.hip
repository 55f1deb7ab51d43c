// Attention backward over packed sequences on MXFP8 operands, gfx950 (CDNA4).
//
// What is computed: LP-FA4 README, section "MXFP8 forward and backward": the backward takes the
// quantized Q, K and V in both hardware orientations, the forward's BF16 output and LSE and the
// output gradient, and returns dQ in BF16 and dK, dV in BF16 or as E4M3 payloads with one E8M0
// scale per 32-element block (head_dim orientation, the quantizer's layout). With tau the
// softmax scale, per sequence and head:
//   P = exp(tau Qd Kd^T - LSE), dP = dO Vd^T, D = rowsum(dO * O), dS = P (dP - D),
//   dV = P^T dO, dK = tau dS^T Qt, dQ = tau dS Kt
// (d: head_dim orientation, t: token orientation: each product takes the orientation whose
// 32-element blocks run along its contraction). P and dS enter the products rounded to BF16.
//
// Kernels (in stream order)
//  * bwd_dequant_kernel: Qd, Qt, Kd, Vd and Kt dequantized once into BF16 copies in the caller's
//    workspace (the main kernels re-read every tile once per 64-row block of the other side).
//    The same launch computes D for every (head, query) into the workspace (16 lanes per row).
//  * bwd_dkdv_kernel: one workgroup = (128 keys of one sequence, head), 8 waves x 16 keys. The
//    keys' K and V fragments and the dK, dV accumulators stay in registers while the workgroup
//    walks the sequence's queries 64 at a time. The epilogue writes BF16, or quantizes each
//    32-element block to MXFP8 with the quantizer's exponent rule (and writes pad scale rows).
//  * bwd_dq_kernel: one workgroup = (128 queries, head), 8 waves x 16 queries, walking the keys.
//    dQ has its own pass instead of atomics from the dK/dV pass, so every result is independent
//    of scheduling; the price is recomputing S and dP.
//
// Matrix instruction: v_mfma_f32_16x16x32_bf16 everywhere, on operands dequantized into BF16
// (an E4M3 code times 2^e has at most 4 significant bits, so the BF16 value is exact inside
// BF16's normal range). The scores are recomputed from these exact
// operands in FP32. Layouts (A lane (g, r): row r, k = 8g..8g+7; B lane (g, c): column c, the
// same k; result lane (g, c): column c, rows 4g..4g+3):
//  * dK/dV pass: S = Q K^T and dP = dO V^T with queries as rows, so lane (g, n) holds key n and
//    queries 4g+i of a 16-query tile. Those values are the A operand of dV = P^T dO and
//    dK = dS^T Qt as they stand, once the 8 k slots of lane group g in a 32-query step are
//    mapped to queries 16(j/4) + 4g + j%4; the B operands (dO and Qt by column, same slot map)
//    come from LDS through transposing reads (ds_read_b64_tr_b16).
//  * dQ pass: S^T = K Q^T and dP^T = V dO^T with keys as rows; lane (g, n) holds query n and keys
//    4g+i, the A operand of dQ = dS Kt under the same map; Kt by column through transposing reads.
// LDS tiles are 64 rows x 128 BF16 (256-byte rows) with 16-byte chunk c of row r stored at
// chunk c ^ (r & 15): a row read (one chunk of 16 rows) and a transposing read (two chunks of 16
// rows) both spread over the banks. Tiles arrive by 16-byte direct-to-LDS loads from the BF16
// copies (double-buffered: the next step's tiles load while the current step computes), and
// fragment reads are issued in groups ahead of the matrix instructions that use them. Each wave
// owns NT 16-row tiles of its own side, and each SIMD runs two waves, so that one wave's softmax
// and LDS waits meet the other's matrix instructions. (Every fragment read from LDS feeds NT
// matrix instructions: at NT = 1 the loop moves twice the LDS bytes per row that NT = 2 does,
// which one wave per SIMD needs, and still runs faster.)
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>
#include <type_traits>

#include "device_common.h"
#include "kernels.h"

namespace lpfa {

namespace {

#define LDS __attribute__((address_space(3)))
typedef short v4s_t __attribute__((ext_vector_type(4)));
typedef unsigned v2u_t __attribute__((ext_vector_type(2)));
typedef unsigned v4u_t __attribute__((ext_vector_type(4)));  // LDS accesses use ext vectors: HIP's
                                                             // uint4 does not bind to LDS references

constexpr int BR = 64;                     // rows of the other side per step (staged tiles)
constexpr int NW = 8;                      // waves per workgroup: two per SIMD
constexpr int WR = 16;                     // rows of the workgroup's own side per wave
constexpr int NT = WR / 16;                // 16-row tiles per wave
constexpr int BO = NW * WR;                // own-side rows per workgroup
constexpr int NTHR = 64 * NW;
constexpr int TILE = BR * 256;             // one staged BF16 tile
constexpr int STAGE = 3 * TILE;            // the three tiles of one step (double-buffered)
constexpr int OFF_VEC = 2 * STAGE;         // dK/dV pass: LSE (log2 units) and D of a step's queries, per buffer
constexpr int LDS_BYTES = 2 * STAGE + 2 * 2 * BR * 4;
constexpr float LOG2E = 1.4426950408889634f;
static_assert(BO * 128 * 4 <= 2 * STAGE, "the FP32 epilogue tile fits in the staging area");

// E8M0 byte -> 2^(b - 127) as a float (b = 0 gives the subnormal 2^-127).
__device__ __forceinline__ float e8m0_f(uint32_t b) {
  return b ? __uint_as_float(b << 23) : __uint_as_float(0x00400000u);
}

// 8 E4M3 codes times one power-of-two scale -> 8 BF16 (the scaled conversion reads only the
// exponent field of `scale`, and 2^-127's field 0 reads as 2^-127).
__device__ __forceinline__ uint4 fp8x8_bf16(uint32_t w0, uint32_t w1, float scale) {
  return make_uint4(__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w0, scale, false)),
                    __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w0, scale, true)),
                    __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w1, scale, false)),
                    __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w1, scale, true)));
}

// Largest i in [0, n) with cu[i] <= row (the sequence that owns padded row `row`; empty
// sequences before it share its offset and are skipped).
__device__ __forceinline__ int find_seq(const int32_t* cu, int n, int row) {
  int lo = 0, hi = n - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (cu[mid] <= row) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// 4 codes of one word, each times its own column scale 2^(b - 127) (an exact ldexp) -> two BF16 pairs
__device__ __forceinline__ uint2 fp8x4_colscaled(uint32_t w, uint32_t s) {
  const float f0 = ldexpf(__builtin_amdgcn_cvt_f32_fp8((int)w, 0), (int)(s & 0xFFu) - 127);
  const float f1 = ldexpf(__builtin_amdgcn_cvt_f32_fp8((int)w, 1), (int)((s >> 8) & 0xFFu) - 127);
  const float f2 = ldexpf(__builtin_amdgcn_cvt_f32_fp8((int)w, 2), (int)((s >> 16) & 0xFFu) - 127);
  const float f3 = ldexpf(__builtin_amdgcn_cvt_f32_fp8((int)w, 3), (int)(s >> 24) - 127);
  return make_uint2(cvt_pk_bf16(f0, f1), cvt_pk_bf16(f2, f3));
}

__device__ __forceinline__ LDS v4u_t* chunk_at(LDS uint8_t* tile, int r, int c) {
  return reinterpret_cast<LDS v4u_t*>(tile + r * 256 + ((c ^ (r & 15)) << 4));
}

// Two floats -> two BF16 (nearest even) in one word, first in the low half (one conversion).
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pk_bf16(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{a, b}, bf16x2_t));
}

__device__ __forceinline__ void wait_vm_all() { __builtin_amdgcn_s_waitcnt(0x0F70); }  // vmcnt(0)

// Stage a 64-row BF16 tile: rows tok0 + r (r clamped to nrows - 1) of head `head` of a
// (tokens, H, 128) BF16 tensor ending at `end`; 16-byte chunk c of row r lands in LDS chunk
// c ^ (r & 15). 16-byte direct-to-LDS loads fill 1 KB (4 rows) each in lane order, so lane L
// fetches the global chunk that belongs at chunk position L % 16 of row L / 16. Wave w loads
// rows 16w .. 16w + 15.
__device__ __forceinline__ void stage_tile(LDS uint8_t* tile, const uint16_t* src, const uint16_t* end,
                                           int64_t tok0, int nrows, int H, int head, int wave, int lane) {
  const uint8_t* b = reinterpret_cast<const uint8_t*>(src + (tok0 * H + head) * 128);
  const int64_t left = reinterpret_cast<const uint8_t*>(end) - b;
  const int n = left <= 0 ? 0 : (left >= 0x7FFFFFFF ? 0x7FFFFFFF : (int)left);
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(b), (short)0, n, 0x00020000);
  constexpr int RW = BR / NW;  // rows per wave
#pragma unroll
  for (int i = 0; i < RW / 4; ++i) {
    const int r = RW * wave + 4 * i + (lane >> 4);
    const int rc = min(r, nrows - 1);
    const uint32_t off = (uint32_t)(rc * H * 256) + 16u * (uint32_t)((lane & 15) ^ (r & 15));
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (LDS void*)(tile + (RW * wave + 4 * i) * 256), 16, off, 0, 0, 0);
  }
}

// ---- operand reads

// Row fragment: row r, k = 32u + 8g .. +7 (chunk 4u + g).
__device__ __forceinline__ v8bf row_frag(LDS uint8_t* tile, int r, int chunk) {
  return __builtin_bit_cast(v8bf, *chunk_at(tile, r, chunk));
}

// Column fragment for a 32-row step s and 16-column tile dt: lane (g, L) receives column
// 16dt + L at rows 32s + 16(j/4) + 4g + j%4 (j = 0..7). In each 16-lane group the transposing
// read gives output lane 4h+i element i of the 8-byte pieces addressed by lanes h, h+4, h+8,
// h+12, so lane L addresses row 4g + L/4 (+16 for the second read) at columns 16dt + 4(L%4) .. +3.
__device__ __forceinline__ v8bf col_frag(LDS uint8_t* tile, int s, int dt, int g, int lam) {
  const int r0 = 32 * s + 4 * g + (lam >> 2);
  const int c = 2 * dt + ((lam >> 1) & 1);
  LDS uint8_t* p0 = tile + r0 * 256 + ((c ^ (r0 & 15)) << 4) + 8 * (lam & 1);
  LDS uint8_t* p1 = p0 + 16 * 256;  // row r0 + 16: same swizzle
  const v2u_t w0 = __builtin_bit_cast(v2u_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16(reinterpret_cast<LDS v4s_t*>(p0)));
  const v2u_t w1 = __builtin_bit_cast(v2u_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16(reinterpret_cast<LDS v4s_t*>(p1)));
  return __builtin_bit_cast(v8bf, make_uint4(w0[0], w0[1], w1[0], w1[1]));
}

__device__ __forceinline__ v4f mfma(v8bf a, v8bf b, v4f c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Ends a scheduling group: the fragment reads written before it are issued together, and the
// matrix instructions that use them follow (one wait for the group instead of one per read).
__device__ __forceinline__ void group_end() { __builtin_amdgcn_sched_barrier(0); }

// (row block, head) of this workgroup in a one-dimensional grid of nblk * H workgroups. Workgroup
// ids are dealt round-robin over the 8 XCDs; with H a multiple of 8, head h runs on XCD h % 8, so
// the other side's tiles of a head, which every row block of that head reads, stay in one L2.
__device__ __forceinline__ void block_head(int nblk, int H, int& blk, int& head) {
  const int L = (int)blockIdx.x;
  if ((H & 7) == 0) {
    const int k = L >> 3;
    head = (L & 7) + 8 * (k / nblk);
    blk = k % nblk;
  } else {
    head = L / nblk;
    blk = L % nblk;
  }
}

// ---- D = rowsum(dO * O)

__device__ __forceinline__ void delta_rows(const BwdParams& p, int64_t gid) {
  const int64_t row = gid >> 4;  // token * H + head
  const int sub = threadIdx.x & 15;
  const bool in = row < p.total_q * p.num_heads;
  float acc = 0.0f;
  if (in) {
    const uint4 o = *reinterpret_cast<const uint4*>(p.out + row * 128 + sub * 8);
    const uint4 d = *reinterpret_cast<const uint4*>(p.dout + row * 128 + sub * 8);
    const uint32_t ow[4] = {o.x, o.y, o.z, o.w}, dw[4] = {d.x, d.y, d.z, d.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) acc += bf16_lo(ow[i]) * bf16_lo(dw[i]) + bf16_hi(ow[i]) * bf16_hi(dw[i]);
  }
#pragma unroll
  for (int o = 1; o < 16; o <<= 1) acc += __shfl_xor(acc, o);
  if (in && sub == 0) {  // stored negated: -D is the initial value of the dP accumulators
    const int64_t tok = row / p.num_heads;
    const int head = (int)(row - tok * p.num_heads);
    p.delta[(int64_t)head * p.total_q + tok] = -acc;
  }
}

// ---- pre-pass: each MX operand dequantized once into a BF16 copy (tokens, H, 128)
// blockIdx.y selects the tensor: 0 Qd, 1 Qt, 2 Kd, 3 Vd, 4 Kt (t: token orientation). A thread
// converts one 8-element chunk of a padded scale row; pad rows have no tokens and are skipped.
__global__ __launch_bounds__(256) void bwd_dequant_kernel(BwdParams p) {
  const int job = blockIdx.y;
  if (job == 5) {  // D = rowsum(dO * O): 16 lanes per (query, head) row; Q's padded rows >= its tokens
    delta_rows(p, (int64_t)blockIdx.x * 256 + threadIdx.x);
    return;
  }
  const bool isq = job < 2, tok_orient = job == 1 || job == 4;
  const uint8_t* pay = job == 0 ? p.q : job == 1 ? p.q_t : job == 2 ? p.k : job == 3 ? p.v : p.k_t;
  const uint8_t* sc = job == 0 ? p.q_scale : job == 1 ? p.q_t_scale : job == 2 ? p.k_scale : job == 3 ? p.v_scale : p.k_t_scale;
  uint16_t* dst = job == 0 ? p.qd16 : job == 1 ? p.qt16 : job == 2 ? p.kd16 : job == 3 ? p.vd16 : p.kt16;
  const int32_t* cu = isq ? p.cu_q : p.cu_k;
  const int32_t* cs = isq ? p.cu_scale_q : p.cu_scale_k;
  const int64_t rows = isq ? p.rows_q : p.rows_k;
  const int H = p.num_heads;
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t srow = gid / (H * 16);
  if (srow >= rows) return;
  const int rem = (int)(gid - srow * H * 16);
  const int head = rem >> 4, c = rem & 15;
  const int seq = find_seq(cs, p.num_seqs, (int)srow);
  const int local = (int)srow - cs[seq];
  if (local >= cu[seq + 1] - cu[seq]) return;  // pad row
  const int64_t off = (((int64_t)cu[seq] + local) * H + head) * 128 + 8 * c;
  const uint2 w = *reinterpret_cast<const uint2*>(pay + off);
  uint4 out;
  if (!tok_orient) {
    out = fp8x8_bf16(w.x, w.y, e8m0_f(sc[(srow * H + head) * 4 + (c >> 2)]));
  } else {
    const int64_t trow = cs[seq] / 32 + local / 32;
    const uint2 sw = *reinterpret_cast<const uint2*>(sc + (trow * H + head) * 128 + 8 * c);
    const uint2 lo = fp8x4_colscaled(w.x, sw.x), hi = fp8x4_colscaled(w.y, sw.y);
    out = make_uint4(lo.x, lo.y, hi.x, hi.y);
  }
  *reinterpret_cast<uint4*>(dst + off) = out;
}

// ---- epilogue: a 64 x 128 FP32 tile in LDS -> BF16 rows, or MXFP8 rows plus scale rows

__device__ __forceinline__ void emit_rows(LDS float* ep, uint8_t* dst, uint8_t* dst_scale, bool mx, int mode,
                                          int64_t tok0, int64_t srow0, int row_base, int rows_valid, int H, int head) {
  const int r = threadIdx.x >> 2, c4 = threadIdx.x & 3;
  const bool valid = row_base + r < rows_valid;
  const LDS v4f* src = reinterpret_cast<const LDS v4f*>(ep + r * 128 + 32 * c4);
  float v[32];
#pragma unroll
  for (int m = 0; m < 8; ++m) {
    const v4f f = src[m];
    v[4 * m] = f[0]; v[4 * m + 1] = f[1]; v[4 * m + 2] = f[2]; v[4 * m + 3] = f[3];
  }
  const int64_t off = ((tok0 + r) * H + head) * 128 + 32 * c4;  // element offset of this quarter row
  if (!mx) {
    if (valid) {
      uint4* d = reinterpret_cast<uint4*>(dst + off * 2);
#pragma unroll
      for (int m = 0; m < 4; ++m)
        d[m] = make_uint4(pk_bf16(v[8 * m], v[8 * m + 1]), pk_bf16(v[8 * m + 2], v[8 * m + 3]),
                          pk_bf16(v[8 * m + 4], v[8 * m + 5]), pk_bf16(v[8 * m + 6], v[8 * m + 7]));
    }
    return;
  }
  uint8_t sbyte = 0x7F;  // pad row of the scale storage
  if (valid) {
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
    const int e = block_exponent(amax, mode);
    const float inv = __uint_as_float((uint32_t)(127 - e) << 23);  // 2^-e, exact (e in [-127, 120])
    uint32_t w[8];
#pragma unroll
    for (int m = 0; m < 8; ++m)
      w[m] = cvt4_e4m3(clamp448(v[4 * m] * inv), clamp448(v[4 * m + 1] * inv), clamp448(v[4 * m + 2] * inv),
                       clamp448(v[4 * m + 3] * inv));
    uint4* d = reinterpret_cast<uint4*>(dst + off);
    d[0] = make_uint4(w[0], w[1], w[2], w[3]);
    d[1] = make_uint4(w[4], w[5], w[6], w[7]);
    sbyte = (uint8_t)(e + 127);
  }
  dst_scale[((srow0 + r) * H + head) * 4 + c4] = sbyte;
}

// accumulators of the wave's 16-row tiles (result layout: lane (g, c) holds rows 16t + 4g + i of
// wave w's WR, column 16dt + c) -> FP32 tile of BO rows in LDS, times `mul`
__device__ __forceinline__ void acc_to_lds(LDS float* ep, const v4f acc[NT][8], float mul, int wave, int g, int n16) {
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int dt = 0; dt < 8; ++dt)
#pragma unroll
      for (int i = 0; i < 4; ++i) ep[(WR * wave + 16 * t + 4 * g + i) * 128 + 16 * dt + n16] = acc[t][dt][i] * mul;
}

// ---- dK, dV
// One workgroup = BO keys of one (sequence, head); wave w owns keys WR w + 16t + n (t < NT): their
// K and V fragments and dK, dV accumulators stay in registers while the workgroup walks the
// sequence's queries 64 at a time. Every fragment read from LDS feeds the wave's NT key tiles. The
// next step's Q, dO and Qt tiles load (into the other buffer) while the current step computes.

__global__ __launch_bounds__(NTHR) void bwd_dkdv_kernel(BwdParams p) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem_dyn[];
  LDS uint8_t* lds = (LDS uint8_t*)smem_dyn;

  const int H = p.num_heads;
  int blk, head;
  block_head((int)(p.rows_k / BO), H, blk, head);
  const int row0 = blk * BO;  // row of K's padded scale storage (sequences are padded to 128)
  const int seq = find_seq(p.cu_scale_k, p.num_seqs, row0);
  const int srow_k = p.cu_scale_k[seq];
  const int k_loc = row0 - srow_k;
  const int kbase = p.cu_k[seq], Lk = p.cu_k[seq + 1] - kbase;
  const int qbase = p.cu_q[seq], Lq = p.cu_q[seq + 1] - qbase;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n16 = lane & 15, g = lane >> 4;

  v4f dv[NT][8], dk[NT][8];
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) dv[t][dt] = dk[t][dt] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

  if (k_loc < Lk && Lq > 0) {
    // this lane's keys (B operand column n16 of tile t): K and V fragments, k = d
    v8bf kf[NT][4], vf[NT][4];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int kr = min(k_loc + WR * wave + 16 * t + n16, Lk - 1);
      const int64_t tk = kbase + kr;
      const uint8_t* kp = p.k + (tk * H + head) * 128 + 8 * g;
      const uint8_t* vp = p.v + (tk * H + head) * 128 + 8 * g;
      const uint8_t* ks = p.k_scale + ((int64_t)(srow_k + kr) * H + head) * 4;
      const uint8_t* vs = p.v_scale + ((int64_t)(srow_k + kr) * H + head) * 4;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const uint2 wk = *reinterpret_cast<const uint2*>(kp + 32 * u);
        const uint2 wv = *reinterpret_cast<const uint2*>(vp + 32 * u);
        kf[t][u] = __builtin_bit_cast(v8bf, fp8x8_bf16(wk.x, wk.y, e8m0_f(ks[u])));
        vf[t][u] = __builtin_bit_cast(v8bf, fp8x8_bf16(wv.x, wv.y, e8m0_f(vs[u])));
      }
    }
    const float c = p.softmax_scale * LOG2E;
    const int nqb = (Lq + BR - 1) / BR;
    const int64_t qelems = p.total_q * H * 128;
    LDS float* vec0 = reinterpret_cast<LDS float*>(lds + OFF_VEC);  // per buffer: [0, 64) LSE, [64, 128) D
    const float* lse_h = p.lse + (int64_t)head * p.total_q + qbase;
    const float* del_h = p.delta + (int64_t)head * p.total_q + qbase;

    // step j's Q, dO and Qt tiles, and its queries' LSE (wave 0) and D (wave 1), into buffer buf
    // (query rows past the sequence read its last row; their P is masked to 0 where it is used)
    auto stage = [&](int j, int buf) {
      const int64_t t0 = qbase + (int64_t)j * BR;
      const int nr = Lq - j * BR;
      LDS uint8_t* b = lds + buf * STAGE;
      stage_tile(b, p.qd16, p.qd16 + qelems, t0, nr, H, head, wave, lane);
      stage_tile(b + TILE, p.dout, p.dout + qelems, t0, nr, H, head, wave, lane);
      stage_tile(b + 2 * TILE, p.qt16, p.qt16 + qelems, t0, nr, H, head, wave, lane);
      if (wave < 2) {
        const float* src = wave == 0 ? lse_h : del_h;
        const auto rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(src), (short)0, Lq * 4, 0x00020000);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (LDS void*)(vec0 + buf * 2 * BR + wave * BR), 4,
                                                 (uint32_t)(min(j * BR + lane, Lq - 1) * 4), 0, 0, 0);
      }
    };
    stage(0, 0);
    wait_vm_all();
    __syncthreads();

    for (int j = 0; j < nqb; ++j) {
      const int buf = j & 1;
      if (j + 1 < nqb) stage(j + 1, buf ^ 1);  // the other buffer: last read in step j - 1
      LDS uint8_t* tq = lds + buf * STAGE;  // Q (head_dim orientation), BF16
      LDS uint8_t* tdo = tq + TILE;         // dO
      LDS uint8_t* tqt = tq + 2 * TILE;     // Q (token orientation)
      LDS float* vec = vec0 + buf * 2 * BR;

      // S and dP: lane (g, n16) holds key 16t + n16 of the wave, queries 16qt + 4g + i. The
      // fragments of query tile qt+1 are read while the matrix instructions of tile qt run; the
      // accumulation chains (S and dP of each key tile) interleave.
      // dP starts from -D of its row, so that it ends as dP - D (the workspace holds -D)
      v4f s[NT][4], dp[NT][4], nd[4];
      v8bf aq[2][4], ao[2][4];
#pragma unroll
      for (int qt = 0; qt < 4; ++qt) nd[qt] = *reinterpret_cast<LDS v4f*>(vec + BR + 16 * qt + 4 * g);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        aq[0][u] = row_frag(tq, n16, 4 * u + g);
        ao[0][u] = row_frag(tdo, n16, 4 * u + g);
      }
#pragma unroll
      for (int qt = 0; qt < 4; ++qt) {
        const int cur = qt & 1;
        if (qt < 3) {
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            aq[cur ^ 1][u] = row_frag(tq, 16 * (qt + 1) + n16, 4 * u + g);
            ao[cur ^ 1][u] = row_frag(tdo, 16 * (qt + 1) + n16, 4 * u + g);
          }
        }
        group_end();
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
          for (int t = 0; t < NT; ++t) {
            s[t][qt] = mfma(aq[cur][u], kf[t][u], u == 0 ? v4f{0.0f, 0.0f, 0.0f, 0.0f} : s[t][qt]);
            dp[t][qt] = mfma(ao[cur][u], vf[t][u], u == 0 ? nd[qt] : dp[t][qt]);
          }
        group_end();
      }
      // the first group of dV/dK operands goes out before the softmax
      v8bf bo[2][4], bq[2][4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        bo[0][i] = col_frag(tdo, 0, i, g, n16);
        bq[0][i] = col_frag(tqt, 0, i, g, n16);
      }
      uint32_t pw[NT][2][4], dw[NT][2][4];
      // LSE in log2 units; on the sequence's last step, +inf past its end (P = 0 there)
      auto probs = [&](auto tail) {
#pragma unroll
        for (int qt = 0; qt < 4; ++qt) {
          const v4f ln = *reinterpret_cast<LDS v4f*>(vec + 16 * qt + 4 * g);
          float lv[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            lv[i] = ln[i] * LOG2E;
            if constexpr (decltype(tail)::value) lv[i] = j * BR + 16 * qt + 4 * g + i < Lq ? lv[i] : __builtin_inff();
          }
#pragma unroll
          for (int t = 0; t < NT; ++t) {
            float pr[4], ds[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              pr[i] = __builtin_amdgcn_exp2f(fmaf(s[t][qt][i], c, -lv[i]));
              ds[i] = pr[i] * dp[t][qt][i];
            }
            pw[t][qt >> 1][2 * (qt & 1)] = pk_bf16(pr[0], pr[1]);
            pw[t][qt >> 1][2 * (qt & 1) + 1] = pk_bf16(pr[2], pr[3]);
            dw[t][qt >> 1][2 * (qt & 1)] = pk_bf16(ds[0], ds[1]);
            dw[t][qt >> 1][2 * (qt & 1) + 1] = pk_bf16(ds[2], ds[3]);
          }
        }
      };
      if (j * BR + BR <= Lq) probs(std::false_type{});
      else probs(std::true_type{});
      // dV += P^T dO, dK += dS^T Qt over 4 groups (32-query half st, d tiles d0..d0+3), the next
      // group's transposed reads going out before the current group's matrix instructions
#pragma unroll
      for (int gi = 0; gi < 4; ++gi) {
        const int st = gi >> 1, d0 = 4 * (gi & 1), cur = gi & 1;
        if (gi < 3) {
          const int st1 = (gi + 1) >> 1, d1 = 4 * ((gi + 1) & 1);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            bo[cur ^ 1][i] = col_frag(tdo, st1, d1 + i, g, n16);
            bq[cur ^ 1][i] = col_frag(tqt, st1, d1 + i, g, n16);
          }
        }
        group_end();
        v8bf ap[NT], ad[NT];
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          ap[t] = __builtin_bit_cast(v8bf, make_uint4(pw[t][st][0], pw[t][st][1], pw[t][st][2], pw[t][st][3]));
          ad[t] = __builtin_bit_cast(v8bf, make_uint4(dw[t][st][0], dw[t][st][1], dw[t][st][2], dw[t][st][3]));
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int t = 0; t < NT; ++t) {
            dv[t][d0 + i] = mfma(ap[t], bo[cur][i], dv[t][d0 + i]);
            dk[t][d0 + i] = mfma(ad[t], bq[cur][i], dk[t][d0 + i]);
          }
        group_end();
      }
      wait_vm_all();
      __syncthreads();
    }
  }

  LDS float* ep = reinterpret_cast<LDS float*>(lds);
  const bool mx = p.mx_dkv != 0;
  acc_to_lds(ep, dv, 1.0f, wave, g, n16);
  __syncthreads();
  for (int r0 = 0; r0 < BO; r0 += NTHR / 4)
    emit_rows(ep + r0 * 128, p.dv, p.dv_scale, mx, p.scaling_mode, kbase + k_loc + r0, srow_k + k_loc + r0, k_loc + r0, Lk,
              H, head);
  __syncthreads();
  acc_to_lds(ep, dk, p.softmax_scale, wave, g, n16);
  __syncthreads();
  for (int r0 = 0; r0 < BO; r0 += NTHR / 4)
    emit_rows(ep + r0 * 128, p.dk, p.dk_scale, mx, p.scaling_mode, kbase + k_loc + r0, srow_k + k_loc + r0, k_loc + r0, Lk,
              H, head);
}

// ---- dQ
// One workgroup = BO queries of one (sequence, head); wave w owns queries WR w + 16t + n (t < NT)
// and walks the keys 64 at a time, double-buffered like the dK/dV pass.

__global__ __launch_bounds__(NTHR) void bwd_dq_kernel(BwdParams p) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem_dyn[];
  LDS uint8_t* lds = (LDS uint8_t*)smem_dyn;

  const int H = p.num_heads;
  int blk, head;
  block_head((int)(p.rows_q / BO), H, blk, head);
  const int row0 = blk * BO;  // row of Q's padded scale storage
  const int seq = find_seq(p.cu_scale_q, p.num_seqs, row0);
  const int srow_q = p.cu_scale_q[seq];
  const int q_loc = row0 - srow_q;
  const int qbase = p.cu_q[seq], Lq = p.cu_q[seq + 1] - qbase;
  const int kbase = p.cu_k[seq], Lk = p.cu_k[seq + 1] - kbase;
  if (q_loc >= Lq) return;  // pad rows only: nothing to write
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n16 = lane & 15, g = lane >> 4;

  v4f dq[NT][8];
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) dq[t][dt] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

  if (Lk > 0) {
    // this lane's queries (B operand column n16 of tile t): Q and dO fragments, k = d
    v8bf qf[NT][4], of[NT][4];
    float l2[NT], dl[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int qv = q_loc + WR * wave + 16 * t + n16;
      const int qr = min(qv, Lq - 1);
      const int64_t tq_ = qbase + qr;
      const uint8_t* qp = p.q + (tq_ * H + head) * 128 + 8 * g;
      const uint8_t* qs = p.q_scale + ((int64_t)(srow_q + qr) * H + head) * 4;
      const uint16_t* op = p.dout + (tq_ * H + head) * 128 + 8 * g;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const uint2 w = *reinterpret_cast<const uint2*>(qp + 32 * u);
        qf[t][u] = __builtin_bit_cast(v8bf, fp8x8_bf16(w.x, w.y, e8m0_f(qs[u])));
        of[t][u] = __builtin_bit_cast(v8bf, *reinterpret_cast<const uint4*>(op + 32 * u));
      }
      l2[t] = qv < Lq ? p.lse[(int64_t)head * p.total_q + tq_] * LOG2E : __builtin_inff();
      dl[t] = p.delta[(int64_t)head * p.total_q + tq_];  // -D
    }
    const float c = p.softmax_scale * LOG2E;
    const int nkb = (Lk + BR - 1) / BR;
    const int64_t kelems = p.total_k * H * 128;

    auto stage = [&](int j, int buf) {
      const int64_t t0 = kbase + (int64_t)j * BR;
      const int nr = Lk - j * BR;
      LDS uint8_t* b = lds + buf * STAGE;
      stage_tile(b, p.kd16, p.kd16 + kelems, t0, nr, H, head, wave, lane);
      stage_tile(b + TILE, p.vd16, p.vd16 + kelems, t0, nr, H, head, wave, lane);
      stage_tile(b + 2 * TILE, p.kt16, p.kt16 + kelems, t0, nr, H, head, wave, lane);
    };
    stage(0, 0);
    wait_vm_all();
    __syncthreads();

    for (int j = 0; j < nkb; ++j) {
      const int buf = j & 1;
      if (j + 1 < nkb) stage(j + 1, buf ^ 1);  // the other buffer: last read in step j - 1
      LDS uint8_t* tk = lds + buf * STAGE;   // K (head_dim orientation), BF16
      LDS uint8_t* tv = tk + TILE;           // V (head_dim orientation)
      LDS uint8_t* tkt = tk + 2 * TILE;      // K (token orientation)
      const int nr = Lk - j * BR;

      // S^T and dP^T: lane (g, n16) holds query 16t + n16 of the wave, keys 16kt + 4g + i
      // (pipelined like the dK/dV pass)
      v4f s[NT][4], dp[NT][4];
      v8bf ak[2][4], av[2][4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        ak[0][u] = row_frag(tk, n16, 4 * u + g);
        av[0][u] = row_frag(tv, n16, 4 * u + g);
      }
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) {
        const int cur = kt & 1;
        if (kt < 3) {
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            ak[cur ^ 1][u] = row_frag(tk, 16 * (kt + 1) + n16, 4 * u + g);
            av[cur ^ 1][u] = row_frag(tv, 16 * (kt + 1) + n16, 4 * u + g);
          }
        }
        group_end();
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
          for (int t = 0; t < NT; ++t) {
            s[t][kt] = mfma(ak[cur][u], qf[t][u], u == 0 ? v4f{0.0f, 0.0f, 0.0f, 0.0f} : s[t][kt]);
            dp[t][kt] = mfma(av[cur][u], of[t][u], u == 0 ? v4f{dl[t], dl[t], dl[t], dl[t]} : dp[t][kt]);
          }
        group_end();
      }
      v8bf bk[2][4];
#pragma unroll
      for (int i = 0; i < 4; ++i) bk[0][i] = col_frag(tkt, 0, i, g, n16);
      uint32_t dw[NT][2][4];
      auto scores_to_ds = [&](auto masked) {
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
#pragma unroll
          for (int t = 0; t < NT; ++t) {
            float ds[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              float pr = __builtin_amdgcn_exp2f(fmaf(s[t][kt][i], c, -l2[t]));
              if constexpr (decltype(masked)::value) pr = 16 * kt + 4 * g + i < nr ? pr : 0.0f;
              ds[i] = pr * dp[t][kt][i];  // dP - D
            }
            dw[t][kt >> 1][2 * (kt & 1)] = pk_bf16(ds[0], ds[1]);
            dw[t][kt >> 1][2 * (kt & 1) + 1] = pk_bf16(ds[2], ds[3]);
          }
      };
      if (nr >= BR) scores_to_ds(std::false_type{});  // a full block: no key mask
      else scores_to_ds(std::true_type{});
#pragma unroll
      for (int gi = 0; gi < 4; ++gi) {
        const int st = gi >> 1, d0 = 4 * (gi & 1), cur = gi & 1;
        if (gi < 3) {
          const int st1 = (gi + 1) >> 1, d1 = 4 * ((gi + 1) & 1);
#pragma unroll
          for (int i = 0; i < 4; ++i) bk[cur ^ 1][i] = col_frag(tkt, st1, d1 + i, g, n16);
        }
        group_end();
        v8bf ad[NT];
#pragma unroll
        for (int t = 0; t < NT; ++t)
          ad[t] = __builtin_bit_cast(v8bf, make_uint4(dw[t][st][0], dw[t][st][1], dw[t][st][2], dw[t][st][3]));
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int t = 0; t < NT; ++t) dq[t][d0 + i] = mfma(ad[t], bk[cur][i], dq[t][d0 + i]);
        group_end();
      }
      wait_vm_all();
      __syncthreads();
    }
  }

  LDS float* ep = reinterpret_cast<LDS float*>(lds);
  acc_to_lds(ep, dq, p.softmax_scale, wave, g, n16);
  __syncthreads();
  uint8_t* dqb = reinterpret_cast<uint8_t*>(p.dq);
  for (int r0 = 0; r0 < BO; r0 += NTHR / 4)
    emit_rows(ep + r0 * 128, dqb, nullptr, false, 0, qbase + q_loc + r0, 0, q_loc + r0, Lq, H, head);
}

}  // namespace

hipError_t launch_attention_bwd(const BwdParams& p, hipStream_t s) {
  // the five operand copies and D in one launch (grid y = job); nothing to contract without
  // both queries and keys (then the main kernels write zeros and read neither)
  const int64_t jobs_rows = p.rows_q > p.rows_k ? p.rows_q : p.rows_k;
  if (p.rows_q > 0 && p.rows_k > 0)
    hipLaunchKernelGGL(bwd_dequant_kernel, dim3((unsigned)((jobs_rows * p.num_heads * 16 + 255) / 256), 6), dim3(256), 0,
                       s, p);
  // more than the default 64 KB of dynamic LDS: a per-kernel, per-device attribute, set once per device
  static std::atomic<uint64_t> configured{0};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const uint64_t bit = dev < 64 ? (uint64_t(1) << dev) : 0;
  if (bit == 0 || !(configured.load(std::memory_order_acquire) & bit)) {
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(&bwd_dkdv_kernel), hipFuncAttributeMaxDynamicSharedMemorySize,
                            LDS_BYTES);
    if (e == hipSuccess)
      e = hipFuncSetAttribute(reinterpret_cast<const void*>(&bwd_dq_kernel), hipFuncAttributeMaxDynamicSharedMemorySize,
                              LDS_BYTES);
    if (e != hipSuccess) return e;
    configured.fetch_or(bit, std::memory_order_acq_rel);
  }
  if (p.rows_k > 0)
    hipLaunchKernelGGL(bwd_dkdv_kernel, dim3((unsigned)(p.rows_k / BO * p.num_heads)), dim3(NTHR), LDS_BYTES, s, p);
  if (p.rows_q > 0)
    hipLaunchKernelGGL(bwd_dq_kernel, dim3((unsigned)(p.rows_q / BO * p.num_heads)), dim3(NTHR), LDS_BYTES, s, p);
  return hipGetLastError();
}

}  // namespace lpfa
