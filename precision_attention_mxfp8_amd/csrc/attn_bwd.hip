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
//  * bwd_delta_kernel: D for every (head, query) into the caller's workspace; 16 lanes per row.
//  * bwd_dkdv_kernel: one workgroup = (64 keys of one sequence, head), 4 waves x 16 keys. The
//    keys' K and V fragments and the dK, dV accumulators stay in registers while the workgroup
//    walks the sequence's queries 64 at a time. The epilogue writes BF16, or quantizes each
//    32-element block to MXFP8 with the quantizer's exponent rule (and writes pad scale rows).
//  * bwd_dq_kernel: one workgroup = (64 queries, head), 4 waves x 16 queries, walking the keys.
//    dQ has its own pass instead of atomics from the dK/dV pass, so every result is independent
//    of scheduling; the price is recomputing S and dP.
//
// Matrix instruction: v_mfma_f32_16x16x32_bf16 everywhere, on operands dequantized into BF16
// while they are staged (an E4M3 code times 2^e has at most 4 significant bits, so the BF16
// value is exact inside BF16's normal range). The scores are recomputed from these exact
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
// rows) both spread over the banks. Staging is single-buffered with the next step's global loads
// issued into registers before the current step's matrix work.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_common.h"
#include "kernels.h"

namespace lpfa {

namespace {

#define LDS __attribute__((address_space(3)))
typedef short v4s_t __attribute__((ext_vector_type(4)));
typedef unsigned v2u_t __attribute__((ext_vector_type(2)));
typedef unsigned v4u_t __attribute__((ext_vector_type(4)));  // LDS accesses use ext vectors: HIP's
                                                             // uint4 does not bind to LDS references

constexpr int BR = 64;                     // rows (keys or queries) per workgroup and per step
constexpr int TILE = BR * 256;             // one BF16 tile
constexpr int OFF_VEC = 3 * TILE;          // dK/dV pass: LSE (log2 units) and D of the step's queries
constexpr int LDS_BYTES = 3 * TILE + 2 * BR * 4;
constexpr float LOG2E = 1.4426950408889634f;
static_assert(BR * 128 * 4 <= 3 * TILE, "the FP32 epilogue tile fits in the staging area");

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

// ---- staging: thread t moves row t/4, columns 32(t%4) .. +31 of a 64-row tile

struct DRaw {  // head_dim orientation: 32 codes + their block's scale byte
  uint4 a, b;
  uint32_t sc;
};
struct TRaw {  // token orientation: 32 codes + one scale byte per column
  uint4 a, b, s0, s1;
};
struct BRaw {  // 32 BF16
  uint4 w[4];
};

__device__ __forceinline__ LDS v4u_t* chunk_at(LDS uint8_t* tile, int r, int c) {
  return reinterpret_cast<LDS v4u_t*>(tile + r * 256 + ((c ^ (r & 15)) << 4));
}

__device__ __forceinline__ v4u_t vu(uint4 x) { return v4u_t{x.x, x.y, x.z, x.w}; }

__device__ __forceinline__ DRaw load_d(const uint8_t* pay, const uint8_t* sc, int64_t tok, int64_t srow, int H,
                                       int head, int c4) {
  const uint4* src = reinterpret_cast<const uint4*>(pay + (tok * H + head) * 128 + 32 * c4);
  DRaw d;
  d.a = src[0];
  d.b = src[1];
  d.sc = sc[(srow * H + head) * 4 + c4];
  return d;
}

__device__ __forceinline__ void store_d(LDS uint8_t* tile, int r, int c4, const DRaw& d) {
  const float s = e8m0_f(d.sc);
  *chunk_at(tile, r, 4 * c4 + 0) = vu(fp8x8_bf16(d.a.x, d.a.y, s));
  *chunk_at(tile, r, 4 * c4 + 1) = vu(fp8x8_bf16(d.a.z, d.a.w, s));
  *chunk_at(tile, r, 4 * c4 + 2) = vu(fp8x8_bf16(d.b.x, d.b.y, s));
  *chunk_at(tile, r, 4 * c4 + 3) = vu(fp8x8_bf16(d.b.z, d.b.w, s));
}

// tok: global token; tscale_row: row of the token-orientation scales (sequence offset / 32 +
// the token's 32-block within the sequence)
__device__ __forceinline__ TRaw load_t(const uint8_t* pay, const uint8_t* tsc, int64_t tok, int64_t tscale_row, int H,
                                       int head, int c4) {
  const uint4* src = reinterpret_cast<const uint4*>(pay + (tok * H + head) * 128 + 32 * c4);
  const uint4* ssrc = reinterpret_cast<const uint4*>(tsc + (tscale_row * H + head) * 128 + 32 * c4);
  TRaw t;
  t.a = src[0];
  t.b = src[1];
  t.s0 = ssrc[0];
  t.s1 = ssrc[1];
  return t;
}

// 4 codes of one word, each times its own column scale -> two BF16 pairs
__device__ __forceinline__ uint2 fp8x4_colscaled(uint32_t w, uint32_t s) {
  const float f0 = __builtin_amdgcn_cvt_f32_fp8((int)w, 0) * e8m0_f(s & 0xFFu);
  const float f1 = __builtin_amdgcn_cvt_f32_fp8((int)w, 1) * e8m0_f((s >> 8) & 0xFFu);
  const float f2 = __builtin_amdgcn_cvt_f32_fp8((int)w, 2) * e8m0_f((s >> 16) & 0xFFu);
  const float f3 = __builtin_amdgcn_cvt_f32_fp8((int)w, 3) * e8m0_f(s >> 24);
  return make_uint2(cvt_pk_bf16(f0, f1), cvt_pk_bf16(f2, f3));
}

__device__ __forceinline__ void store_t(LDS uint8_t* tile, int r, int c4, const TRaw& t) {
  const uint32_t w[8] = {t.a.x, t.a.y, t.a.z, t.a.w, t.b.x, t.b.y, t.b.z, t.b.w};
  const uint32_t s[8] = {t.s0.x, t.s0.y, t.s0.z, t.s0.w, t.s1.x, t.s1.y, t.s1.z, t.s1.w};
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const uint2 lo = fp8x4_colscaled(w[2 * m], s[2 * m]);
    const uint2 hi = fp8x4_colscaled(w[2 * m + 1], s[2 * m + 1]);
    *chunk_at(tile, r, 4 * c4 + m) = v4u_t{lo.x, lo.y, hi.x, hi.y};
  }
}

__device__ __forceinline__ BRaw load_b(const uint16_t* src, int64_t tok, int H, int head, int c4) {
  const uint4* p = reinterpret_cast<const uint4*>(src + (tok * H + head) * 128 + 32 * c4);
  BRaw b;
#pragma unroll
  for (int m = 0; m < 4; ++m) b.w[m] = p[m];
  return b;
}

__device__ __forceinline__ void store_b(LDS uint8_t* tile, int r, int c4, const BRaw& b) {
#pragma unroll
  for (int m = 0; m < 4; ++m) *chunk_at(tile, r, 4 * c4 + m) = vu(b.w[m]);
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

// ---- D = rowsum(dO * O)

__global__ __launch_bounds__(256) void bwd_delta_kernel(BwdParams p) {
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
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
  if (in && sub == 0) {
    const int64_t tok = row / p.num_heads;
    const int head = (int)(row - tok * p.num_heads);
    p.delta[(int64_t)head * p.total_q + tok] = acc;
  }
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
        d[m] = make_uint4(cvt_pk_bf16(v[8 * m], v[8 * m + 1]), cvt_pk_bf16(v[8 * m + 2], v[8 * m + 3]),
                          cvt_pk_bf16(v[8 * m + 4], v[8 * m + 5]), cvt_pk_bf16(v[8 * m + 6], v[8 * m + 7]));
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

// accumulators (result layout: lane (g, c) holds rows 4g+i of wave w's 16, column 16dt + c)
// -> FP32 tile in LDS, times `mul`
__device__ __forceinline__ void acc_to_lds(LDS float* ep, const v4f acc[8], float mul, int wave, int g, int n16) {
#pragma unroll
  for (int dt = 0; dt < 8; ++dt)
#pragma unroll
    for (int i = 0; i < 4; ++i) ep[(16 * wave + 4 * g + i) * 128 + 16 * dt + n16] = acc[dt][i] * mul;
}

// ---- dK, dV

__global__ __launch_bounds__(256) void bwd_dkdv_kernel(BwdParams p) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[LDS_BYTES];
  LDS uint8_t* lds = (LDS uint8_t*)smem;
  LDS uint8_t* tq = lds;             // Q (head_dim orientation), BF16
  LDS uint8_t* tdo = lds + TILE;     // dO
  LDS uint8_t* tqt = lds + 2 * TILE; // Q (token orientation), BF16
  LDS float* vec = reinterpret_cast<LDS float*>(lds + OFF_VEC);  // [0, 64): LSE * log2 e; [64, 128): D

  const int H = p.num_heads, head = blockIdx.y;
  const int row0 = blockIdx.x * BR;  // row of K's padded scale storage
  const int seq = find_seq(p.cu_scale_k, p.num_seqs, row0);
  const int srow_k = p.cu_scale_k[seq];
  const int k_loc = row0 - srow_k;
  const int kbase = p.cu_k[seq], Lk = p.cu_k[seq + 1] - kbase;
  const int qbase = p.cu_q[seq], Lq = p.cu_q[seq + 1] - qbase;
  const int srow_q = p.cu_scale_q[seq];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n16 = lane & 15, g = lane >> 4;
  const int r = tid >> 2, c4 = tid & 3;

  v4f dv[8], dk[8];
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) dv[dt] = dk[dt] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

  if (k_loc < Lk && Lq > 0) {
    // this lane's key (B operand column n16 of the wave's 16): K and V fragments, k = d
    const int kr = min(k_loc + 16 * wave + n16, Lk - 1);
    const int64_t tk = kbase + kr;
    v8bf kf[4], vf[4];
    {
      const uint8_t* kp = p.k + (tk * H + head) * 128 + 8 * g;
      const uint8_t* vp = p.v + (tk * H + head) * 128 + 8 * g;
      const uint8_t* ks = p.k_scale + ((int64_t)(srow_k + kr) * H + head) * 4;
      const uint8_t* vs = p.v_scale + ((int64_t)(srow_k + kr) * H + head) * 4;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const uint2 wk = *reinterpret_cast<const uint2*>(kp + 32 * u);
        const uint2 wv = *reinterpret_cast<const uint2*>(vp + 32 * u);
        kf[u] = __builtin_bit_cast(v8bf, fp8x8_bf16(wk.x, wk.y, e8m0_f(ks[u])));
        vf[u] = __builtin_bit_cast(v8bf, fp8x8_bf16(wv.x, wv.y, e8m0_f(vs[u])));
      }
    }
    const float c = p.softmax_scale * LOG2E;
    const int nqb = (Lq + BR - 1) / BR;

    DRaw rq;
    BRaw rdo;
    TRaw rqt;
    float rl2 = 0.0f, rdl = 0.0f;
    auto load_step = [&](int j) {
      const int qr = min(j * BR + r, Lq - 1);
      const int64_t tq_ = qbase + qr;
      rq = load_d(p.q, p.q_scale, tq_, srow_q + qr, H, head, c4);
      rdo = load_b(p.dout, tq_, H, head, c4);
      rqt = load_t(p.q_t, p.q_t_scale, tq_, srow_q / 32 + qr / 32, H, head, c4);
      if (tid < BR) {
        const int qv = j * BR + tid;
        const int64_t t2 = qbase + min(qv, Lq - 1);
        rl2 = qv < Lq ? p.lse[(int64_t)head * p.total_q + t2] * LOG2E : __builtin_inff();
        rdl = qv < Lq ? p.delta[(int64_t)head * p.total_q + t2] : 0.0f;
      }
    };
    load_step(0);
    for (int j = 0; j < nqb; ++j) {
      store_d(tq, r, c4, rq);
      store_b(tdo, r, c4, rdo);
      store_t(tqt, r, c4, rqt);
      if (tid < BR) {
        vec[tid] = rl2;
        vec[BR + tid] = rdl;
      }
      __syncthreads();
      if (j + 1 < nqb) load_step(j + 1);

      // S and dP: lane (g, n16) holds key n16 of the wave, queries 16qt + 4g + i
      v4f s[4], dp[4];
#pragma unroll
      for (int qt = 0; qt < 4; ++qt) {
        s[qt] = dp[qt] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          s[qt] = mfma(row_frag(tq, 16 * qt + n16, 4 * u + g), kf[u], s[qt]);
          dp[qt] = mfma(row_frag(tdo, 16 * qt + n16, 4 * u + g), vf[u], dp[qt]);
        }
      }
      uint32_t pw[2][4], dw[2][4];
#pragma unroll
      for (int qt = 0; qt < 4; ++qt) {
        const v4f lv = *reinterpret_cast<LDS v4f*>(vec + 16 * qt + 4 * g);
        const v4f dv4 = *reinterpret_cast<LDS v4f*>(vec + BR + 16 * qt + 4 * g);
        float pr[4], ds[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          pr[i] = __builtin_amdgcn_exp2f(fmaf(s[qt][i], c, -lv[i]));
          ds[i] = pr[i] * (dp[qt][i] - dv4[i]);
        }
        pw[qt >> 1][2 * (qt & 1)] = cvt_pk_bf16(pr[0], pr[1]);
        pw[qt >> 1][2 * (qt & 1) + 1] = cvt_pk_bf16(pr[2], pr[3]);
        dw[qt >> 1][2 * (qt & 1)] = cvt_pk_bf16(ds[0], ds[1]);
        dw[qt >> 1][2 * (qt & 1) + 1] = cvt_pk_bf16(ds[2], ds[3]);
      }
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        const v8bf ap = __builtin_bit_cast(v8bf, make_uint4(pw[st][0], pw[st][1], pw[st][2], pw[st][3]));
        const v8bf ad = __builtin_bit_cast(v8bf, make_uint4(dw[st][0], dw[st][1], dw[st][2], dw[st][3]));
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) {
          dv[dt] = mfma(ap, col_frag(tdo, st, dt, g, n16), dv[dt]);
          dk[dt] = mfma(ad, col_frag(tqt, st, dt, g, n16), dk[dt]);
        }
      }
      __syncthreads();
    }
  }

  LDS float* ep = reinterpret_cast<LDS float*>(lds);
  acc_to_lds(ep, dv, 1.0f, wave, g, n16);
  __syncthreads();
  emit_rows(ep, p.dv, p.dv_scale, p.mx_dkv != 0, p.scaling_mode, kbase + k_loc, srow_k + k_loc, k_loc, Lk, H, head);
  __syncthreads();
  acc_to_lds(ep, dk, p.softmax_scale, wave, g, n16);
  __syncthreads();
  emit_rows(ep, p.dk, p.dk_scale, p.mx_dkv != 0, p.scaling_mode, kbase + k_loc, srow_k + k_loc, k_loc, Lk, H, head);
}

// ---- dQ

__global__ __launch_bounds__(256) void bwd_dq_kernel(BwdParams p) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[LDS_BYTES];
  LDS uint8_t* lds = (LDS uint8_t*)smem;
  LDS uint8_t* tk = lds;              // K (head_dim orientation), BF16
  LDS uint8_t* tv = lds + TILE;       // V (head_dim orientation)
  LDS uint8_t* tkt = lds + 2 * TILE;  // K (token orientation)

  const int H = p.num_heads, head = blockIdx.y;
  const int row0 = blockIdx.x * BR;  // row of Q's padded scale storage
  const int seq = find_seq(p.cu_scale_q, p.num_seqs, row0);
  const int srow_q = p.cu_scale_q[seq];
  const int q_loc = row0 - srow_q;
  const int qbase = p.cu_q[seq], Lq = p.cu_q[seq + 1] - qbase;
  const int kbase = p.cu_k[seq], Lk = p.cu_k[seq + 1] - kbase;
  const int srow_k = p.cu_scale_k[seq];
  if (q_loc >= Lq) return;  // pad rows only: nothing to write
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n16 = lane & 15, g = lane >> 4;
  const int r = tid >> 2, c4 = tid & 3;

  v4f dq[8];
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) dq[dt] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

  if (Lk > 0) {
    // this lane's query (B operand column n16 of the wave's 16): Q and dO fragments, k = d
    const int qv = q_loc + 16 * wave + n16;
    const int qr = min(qv, Lq - 1);
    const int64_t tq_ = qbase + qr;
    v8bf qf[4], of[4];
    {
      const uint8_t* qp = p.q + (tq_ * H + head) * 128 + 8 * g;
      const uint8_t* qs = p.q_scale + ((int64_t)(srow_q + qr) * H + head) * 4;
      const uint16_t* op = p.dout + (tq_ * H + head) * 128 + 8 * g;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const uint2 w = *reinterpret_cast<const uint2*>(qp + 32 * u);
        qf[u] = __builtin_bit_cast(v8bf, fp8x8_bf16(w.x, w.y, e8m0_f(qs[u])));
        of[u] = __builtin_bit_cast(v8bf, *reinterpret_cast<const uint4*>(op + 32 * u));
      }
    }
    const float l2 = qv < Lq ? p.lse[(int64_t)head * p.total_q + tq_] * LOG2E : __builtin_inff();
    const float dl = p.delta[(int64_t)head * p.total_q + tq_];
    const float c = p.softmax_scale * LOG2E;
    const int nkb = (Lk + BR - 1) / BR;

    DRaw rk, rv;
    TRaw rkt;
    auto load_step = [&](int j) {
      const int kr = min(j * BR + r, Lk - 1);
      const int64_t t = kbase + kr;
      rk = load_d(p.k, p.k_scale, t, srow_k + kr, H, head, c4);
      rv = load_d(p.v, p.v_scale, t, srow_k + kr, H, head, c4);
      rkt = load_t(p.k_t, p.k_t_scale, t, srow_k / 32 + kr / 32, H, head, c4);
    };
    load_step(0);
    for (int j = 0; j < nkb; ++j) {
      store_d(tk, r, c4, rk);
      store_d(tv, r, c4, rv);
      store_t(tkt, r, c4, rkt);
      __syncthreads();
      if (j + 1 < nkb) load_step(j + 1);

      // S^T and dP^T: lane (g, n16) holds query n16 of the wave, keys 16kt + 4g + i
      v4f s[4], dp[4];
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) {
        s[kt] = dp[kt] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          s[kt] = mfma(row_frag(tk, 16 * kt + n16, 4 * u + g), qf[u], s[kt]);
          dp[kt] = mfma(row_frag(tv, 16 * kt + n16, 4 * u + g), of[u], dp[kt]);
        }
      }
      uint32_t dw[2][4];
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) {
        float ds[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const bool kin = j * BR + 16 * kt + 4 * g + i < Lk;
          const float pr = kin ? __builtin_amdgcn_exp2f(fmaf(s[kt][i], c, -l2)) : 0.0f;
          ds[i] = pr * (dp[kt][i] - dl);
        }
        dw[kt >> 1][2 * (kt & 1)] = cvt_pk_bf16(ds[0], ds[1]);
        dw[kt >> 1][2 * (kt & 1) + 1] = cvt_pk_bf16(ds[2], ds[3]);
      }
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        const v8bf ad = __builtin_bit_cast(v8bf, make_uint4(dw[st][0], dw[st][1], dw[st][2], dw[st][3]));
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) dq[dt] = mfma(ad, col_frag(tkt, st, dt, g, n16), dq[dt]);
      }
      __syncthreads();
    }
  }

  LDS float* ep = reinterpret_cast<LDS float*>(lds);
  acc_to_lds(ep, dq, p.softmax_scale, wave, g, n16);
  __syncthreads();
  emit_rows(ep, reinterpret_cast<uint8_t*>(p.dq), nullptr, false, 0, qbase + q_loc, 0, q_loc, Lq, H, head);
}

}  // namespace

hipError_t launch_attention_bwd(const BwdParams& p, hipStream_t s) {
  const int64_t rows = p.total_q * p.num_heads;
  if (rows > 0)
    hipLaunchKernelGGL(bwd_delta_kernel, dim3((unsigned)((rows * 16 + 255) / 256)), dim3(256), 0, s, p);
  if (p.rows_k > 0)
    hipLaunchKernelGGL(bwd_dkdv_kernel, dim3((unsigned)(p.rows_k / BR), (unsigned)p.num_heads), dim3(256), 0, s, p);
  if (p.rows_q > 0)
    hipLaunchKernelGGL(bwd_dq_kernel, dim3((unsigned)(p.rows_q / BR), (unsigned)p.num_heads), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace lpfa
