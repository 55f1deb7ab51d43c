// Fused noncausal head_dim-128 attention forward over packed sequences, gfx950 (CDNA4).
//
// What is computed: LP-FA4 README (introduction; section "MXFP8 forward and backward"):
// MXFP8 Q/K, noncausal MHA, (out, lse); FastVideo fp8-PV PR: V is BF16 or an unscaled E4M3
// cast read with dequant scale 1.0, output BF16; vLLM unit-descale PR: optional per-tensor
// descales, a missing one read as 1.0 through the same arithmetic.
//
// Work split: one workgroup = one (sequence, head, 128-query tile); 4 waves x 32 queries, one
// wave per SIMD. Keys are processed in blocks of 128.
//
// Matrix instructions and register layouts
//  * Scores are computed transposed, S^T = K Q^T, with v_mfma_scale_f32_16x16x128_f8f6f4: one
//    instruction covers head_dim = 128 for 16 keys x 16 queries and takes the E8M0 block scales
//    as per-lane operands (lane 16b + r supplies block b of row r). Per-tensor mode uses 127 (1.0).
//  * Lane (n, g) of the result holds query n and keys 16*mt + 4*g + i, so row maxima and sums
//    are in-lane plus two cross-lane steps, and the probabilities are already the B operand of
//    O^T = V^T P^T once the K slots of the P V instruction are mapped to the keys that the
//    score layout produced (key 16*(j/4) + 4*g + j%4 sits in byte/element j of lane group g).
//      fp8 PV:  v_mfma_f32_16x16x128_f8f6f4 (scale 1.0), one instruction per 16(d) x 16(q) tile;
//      bf16 PV: v_mfma_f32_16x16x32_bf16, four per tile.
//  * V stays in natural (key, d) order in LDS and is read transposed with ds_read_b64_tr_b8 /
//    ds_read_b64_tr_b16: inside each 16-lane group the transposing read hands output lane 8h+i
//    (b8) byte i of the chunks addressed by lanes h, h+2, .., h+14 (b16: output lane 4h+i gets
//    element i of lanes h, h+4, h+8, h+12), so each lane addresses the key row whose value it
//    must contribute.
//
// Data movement
//  * K, its scales and V move global -> LDS with 16-byte (4-byte for scales) direct-to-LDS loads
//    (global_load_lds): no VGPR staging. Each instruction fills 1 KB of LDS in lane order, so
//    the XOR swizzles are applied by choosing which global chunk each lane fetches.
//      K row r: 16-byte chunk c stored at c ^ (r & 7)          (conflict-free score operand reads)
//      V fp8 row r: chunk c stored at c ^ ((r & 3) | ((r >> 2) & 4))   (conflict-free tr_b8 reads)
//      V bf16 row r: chunk c stored at c ^ (2 * (r & 3))             (conflict-free tr_b16 reads)
//  * K is double-buffered and V triple-buffered so that the loads for blocks j+2 (K) and j+1 (V)
//    are issued a full iteration before they are needed.
//
// Pipeline (iteration j): the score instructions for block j+1 and the P V instructions for
// block j-1 overlap the softmax VALU work of block j. In the BF16 mode the running maximum is
// lazy (see Lazy) and O is normalised by the sum of the probabilities as rounded for the P V
// instruction (summed on the matrix core against an all-ones tile), so a dominant probability's
// rounding cancels; in the FP8 mode the maximum is exact and O uses the FP32 sum. LSE always
// uses the unrounded FP32 sum.
//
// Precision guard: the FP8 matrix instructions sum each group of 8 consecutive products on a
// fixed-point grid 13 bits below the group's largest product (truncating) and the groups in
// FP32, so a score carries an absolute error up to ~2^-12 of the largest product in its row.
// Before each key block the kernel bounds c * max|q| * max|k| (c = softmax_scale * log2 e *
// descales; in MX mode from the E8M0 scales: block maxima lie in (224, 448] * 2^e; in
// per-tensor mode from the E4M3 range 448). Above GUARD_LOG2 = 16 the block's scores are
// computed instead with v_mfma_f32_16x16x32_bf16 on exactly dequantized operands
// (v_cvt_scalef32_pk_bf16_fp8), whose accumulation is FP32-exact in practice. Typical N(0,1)
// data stays on the FP8 path; rows dominated by outliers take the BF16 path.
//
// Workgroup ids are remapped so that consecutive tiles of one (sequence, head) land on the same
// XCD (ids are dealt round-robin over the 8 XCDs), sharing K/V in that XCD's L2.
#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>
#include <stdint.h>

#include <atomic>

#include "device_common.h"
#include "kernels.h"

namespace lpfa {

namespace {

constexpr int BM = 128;  // queries per workgroup
constexpr int BN = 128;  // keys per block
constexpr float LN2 = 0.69314718055994530942f;
constexpr float GUARD_LOG2 = 16.0f;
// Stale-maximum slack of the online softmax, in log2 units. BF16 probabilities may be taken
// against a maximum up to 8 below the running one (P <= 2^8); E4M3 probabilities are rounded
// against the exact running maximum, so that the largest probability is exactly 1 and the
// rounding of the others tracks a rounding against the final maximum as closely as a single
// pass allows (a stale maximum shifts every probability by a non-power-of-two factor and
// decorrelates the E4M3 rounding).
template <bool FP8V>
struct Lazy { static constexpr float LOG2 = FP8V ? 0.0f : 8.0f; };

typedef int v2i_t __attribute__((ext_vector_type(2)));
typedef short v4s_t __attribute__((ext_vector_type(4)));
typedef __bf16 v2bf_t __attribute__((ext_vector_type(2)));
typedef unsigned v2u_t __attribute__((ext_vector_type(2)));
// BF16 operands are always assembled from whole 32-bit words: building them element by element
// from 16-bit values lets the compiler repack halves (it has emitted a repack that dropped the
// second register of a transposed read).
#define LDS_PTR(T, p) ((__attribute__((address_space(3))) T*)(p))
#define LDS __attribute__((address_space(3)))
// LDS byte address (32-bit) -> typed LDS pointer, so offsets fold into the DS immediate field.
template <typename T>
__device__ __forceinline__ LDS T* lds_at(uint32_t byte_addr) {
  return reinterpret_cast<LDS T*>(static_cast<uintptr_t>(byte_addr));
}

template <bool FP8V>
struct Lay {
  static constexpr int K_BYTES = BN * 128;
  static constexpr int KSC_BYTES = BN * 4;
  static constexpr int V_BYTES = FP8V ? BN * 128 : BN * 256;
  static constexpr int OFF_K = 0;                       // 2 buffers
  static constexpr int OFF_KSC = 2 * K_BYTES;           // 2 buffers
  static constexpr int OFF_V = OFF_KSC + 2 * KSC_BYTES; // 3 buffers
  static constexpr int TOTAL = OFF_V + 3 * V_BYTES + 16;  // + guard reduction slots
};

__device__ __forceinline__ uint4 ldg16(const void* p) { return *reinterpret_cast<const uint4*>(p); }
__device__ __forceinline__ uint2 ldg8(const void* p) { return *reinterpret_cast<const uint2*>(p); }

typedef unsigned v4u_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ v8i make_v8i(v4u_t a, v4u_t b) {
  v8i r;
  r[0] = (int)a[0]; r[1] = (int)a[1]; r[2] = (int)a[2]; r[3] = (int)a[3];
  r[4] = (int)b[0]; r[5] = (int)b[1]; r[6] = (int)b[2]; r[7] = (int)b[3];
  return r;
}

__device__ __forceinline__ v8i make_v8i(uint4 a, uint4 b) {
  v8i r;
  r[0] = (int)a.x; r[1] = (int)a.y; r[2] = (int)a.z; r[3] = (int)a.w;
  r[4] = (int)b.x; r[5] = (int)b.y; r[6] = (int)b.z; r[7] = (int)b.w;
  return r;
}

// 8 E4M3 codes -> 8 BF16 values times a power-of-two scale (exact: the scaled conversion uses
// only the exponent of `scale`).
__device__ __forceinline__ v8bf fp8x8_to_bf16(uint32_t w0, uint32_t w1, float scale) {
  const uint32_t a = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w0, scale, false));
  const uint32_t b = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w0, scale, true));
  const uint32_t c = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w1, scale, false));
  const uint32_t d = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w1, scale, true));
  return __builtin_bit_cast(v8bf, make_uint4(a, b, c, d));
}

// E8M0 byte -> float 2^(b-127) for b in 1..254 (b = 0 gives 0.0, whose exponent field the
// scaled conversion reads as 2^-127).
__device__ __forceinline__ float e8m0_to_float(uint32_t b) { return __uint_as_float(b << 23); }

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int s = 1; s < 64; s <<= 1) x = fmaxf(x, __shfl_xor(x, s));
  return x;
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t x) {
#pragma unroll
  for (int s = 1; s < 64; s <<= 1) x = max(x, (uint32_t)__shfl_xor((int)x, s));
  return x;
}

__device__ __forceinline__ void wait_vm_all() { __builtin_amdgcn_s_waitcnt(0x0F70); }  // vmcnt(0)

template <bool MX, bool FP8V>
struct Attn {
  using L = Lay<FP8V>;

  // ---- per-workgroup constants ----
  const AttnParams& p;
  uint8_t* lds;
  uint32_t lds_base;         // LDS byte address of the dynamic allocation
  int seq, head, H, Lk, nb;
  int lane, wave, n16, g;
  const uint8_t* kbase;      // key row 0 of this (sequence, head)
  const uint8_t* vbase;      // value row 0 (bytes)
  int64_t k_st_b, v_st_b;    // row strides in bytes
  const uint8_t* ksc_base;   // scale word of key row 0 of this (sequence, head)
  float c;                   // softmax_scale * log2(e) * qd * kd

  // ---- per-wave state ----
  v8i qf[2];
  int qsc[2];
  float qbound;              // max |q| bound of the wave's queries
  const uint8_t* qrow[2];    // this lane's query rows (nullptr past the end)
  uint32_t qsw[2];           // their E8M0 scale words
  float m_run[2], l_run[2];
  v4f o[8][2];
  v4f o_sum[2];              // sum over keys of the rounded probabilities (ones tile of V^T)

  __device__ Attn(const AttnParams& p_, uint8_t* lds_)
      : p(p_), lds(lds_), lds_base((uint32_t)(uintptr_t)(LDS uint8_t*)lds_) {}

  // ---------------------------------------------------------------- global -> LDS
  // Per-lane byte offsets of the rows each lane fetches, relative to the block's first row
  // (uniform base, so the loads use the scalar-base addressing form). Rows past the end of
  // the sequence are clamped to its last row (those keys are masked, their V rows get P = 0).
  __device__ __forceinline__ uint32_t k_lane_off(int i, int kb, bool clamp) const {
    const int r = 8 * (4 * wave + i) + (lane >> 3);
    const int c = (lane & 7) ^ (lane >> 3);
    const int row = clamp ? min(r, Lk - 1 - kb) : r;
    return (uint32_t)(row * (int)k_st_b) + 16u * c;
  }
  __device__ __forceinline__ uint32_t v_lane_off(int i, int kb, bool clamp) const {
    int r, c;
    if (FP8V) {
      r = 8 * (4 * wave + i) + (lane >> 3);
      c = (lane & 7) ^ ((r & 3) | ((r >> 2) & 4));
    } else {
      r = 4 * (8 * wave + i) + (lane >> 4);
      c = (lane & 15) ^ (2 * (r & 3));
    }
    const int row = clamp ? min(r, Lk - 1 - kb) : r;
    return (uint32_t)(row * (int)v_st_b) + 16u * c;
  }

  __device__ __forceinline__ void dma_k(int blk, int buf) {
    const int kb = blk * BN;
    const bool clamp = kb + BN > Lk;
    const uint8_t* base = kbase + (int64_t)kb * k_st_b;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int R = 4 * wave + i;               // 1 KB region = 8 key rows
      __builtin_amdgcn_global_load_lds(base + k_lane_off(i, kb, clamp),
                                       LDS_PTR(void, lds + L::OFF_K + buf * L::K_BYTES + R * 1024), 16, 0, 0);
    }
    if (MX && wave < 2) {
      const int row = min(kb + 64 * wave + lane, Lk - 1);
      __builtin_amdgcn_global_load_lds(ksc_base + (uint32_t)(row * H * 4),
                                       LDS_PTR(void, lds + L::OFF_KSC + buf * L::KSC_BYTES + wave * 256), 4, 0, 0);
    }
  }

  __device__ __forceinline__ void dma_v(int blk, int buf) {
    const int kb = blk * BN;
    const bool clamp = kb + BN > Lk;
    const uint8_t* base = vbase + (int64_t)kb * v_st_b;
    constexpr int N = FP8V ? 4 : 8;             // 1 KB regions per wave
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int R = N * wave + i;
      __builtin_amdgcn_global_load_lds(base + v_lane_off(i, kb, clamp),
                                       LDS_PTR(void, lds + L::OFF_V + buf * L::V_BYTES + R * 1024), 16, 0, 0);
    }
  }

  // ---------------------------------------------------------------- precision guard
  // True when the whole tile may use the FP8 score path: c * max|q| * max|k| <= GUARD_LOG2 with
  // max|q| over the workgroup's queries and max|k| over all keys of the (sequence, head). In MX
  // mode both bounds come from the E8M0 scales (block maxima lie in (224, 448] * 2^e); in
  // per-tensor mode |q| is read from the codes and |k| is bounded by the E4M3 range.
  __device__ __forceinline__ bool fp8_scores_ok_tile(float* red) {
    float kbound = 448.0f;
    if (MX) {
      uint32_t m = 0;
      for (int row = threadIdx.x; row < Lk; row += 256) {
        const uint32_t w = *reinterpret_cast<const uint32_t*>(ksc_base + (int64_t)row * H * 4);
        m = max(m, max(max(w & 0xFF, (w >> 8) & 0xFF), max((w >> 16) & 0xFF, w >> 24)));
      }
      kbound = 448.0f * e8m0_to_float(wave_max_u32(m));
    }
    float b = c * qbound * kbound;       // per wave
    if (lane == 0) red[wave] = b;
    __syncthreads();
    b = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    __syncthreads();
    return b <= GUARD_LOG2;
  }

  // ---------------------------------------------------------------- scores
  __device__ __forceinline__ void scores_fp8(int buf, v4f s[8][2]) {
    const uint32_t kt = lds_base + L::OFF_K + buf * L::K_BYTES;
    LDS const uint32_t* ksc = lds_at<const uint32_t>(lds_base + L::OFF_KSC + buf * L::KSC_BYTES);
    LDS const v4u_t* k_a = lds_at<const v4u_t>(kt + n16 * 128 + ((g ^ (n16 & 7)) << 4));
    LDS const v4u_t* k_b = lds_at<const v4u_t>(kt + n16 * 128 + (((4 + g) ^ (n16 & 7)) << 4));
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) {
      const v8i kf = make_v8i(k_a[mt * 128], k_b[mt * 128]);
      const int ks = MX ? (int)((ksc[16 * mt + n16] >> (8 * g)) & 0xFFu) : 127;
#pragma unroll
      for (int nt = 0; nt < 2; ++nt)
        s[mt][nt] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(kf, qf[nt], v4f{0.0f, 0.0f, 0.0f, 0.0f},
                                                                     0, 0, 0, ks, 0, qsc[nt]);
    }
  }

  __device__ __forceinline__ void scores_bf16(int buf, v4f s[8][2]) {
    const uint8_t* kt = lds + L::OFF_K + buf * L::K_BYTES;
    const uint32_t* ksc = reinterpret_cast<const uint32_t*>(lds + L::OFF_KSC + buf * L::KSC_BYTES);
    v8bf qb[2][4];  // B operand: lane (n, g) holds d = 32u + 8g + 0..7, exactly dequantized
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        uint2 w = make_uint2(0, 0);
        if (qrow[nt] != nullptr) w = ldg8(qrow[nt] + 32 * u + 8 * g);
        qb[nt][u] = fp8x8_to_bf16(w.x, w.y, e8m0_to_float((qsw[nt] >> (8 * u)) & 0xFFu));
      }
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) {
      const int r = 16 * mt + n16;
      const uint32_t sw = MX ? ksc[r] : 0x7F7F7F7Fu;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int chunk = (2 * u + (g >> 1)) ^ (n16 & 7);
        const uint2 w = *reinterpret_cast<const uint2*>(kt + r * 128 + chunk * 16 + 8 * (g & 1));
        const v8bf kf = fp8x8_to_bf16(w.x, w.y, e8m0_to_float((sw >> (8 * u)) & 0xFFu));
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
          s[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qb[nt][u], u == 0 ? v4f{0.0f, 0.0f, 0.0f, 0.0f} : s[mt][nt], 0, 0, 0);
      }
    }
  }

  // ---------------------------------------------------------------- P V
  // P fragments: fp8 mode one v8i per query tile (byte 4*mt + i = key 16*mt + 4*g + i);
  // bf16 mode 4 chunks of 32 keys, 4 words each (element j = key 32u + 16*(j/4) + 4*g + j%4).
  struct PFrag {
    v8i f8[2];
    uint32_t b16w[4][2][4];
  };

  // O^T d tile dt += V(j-1)^T P(j-1)^T, V read transposed from the natural-layout LDS tile.
  // v_lane: this lane's LDS byte address inside the V buffer for d tile 0 (see pv()).
  __device__ __forceinline__ void pv_tile(uint32_t v_lane, int dt, int jj, const PFrag& pf) {
    if (FP8V) {
      LDS v2i_t* base = lds_at<v2i_t>(v_lane + ((dt ^ jj) << 4));
      v8i vf;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const v2i_t w = __builtin_amdgcn_ds_read_tr8_b64_v2i32(base + r * 512);  // + r * 4096 bytes
        vf[2 * r] = w[0];
        vf[2 * r + 1] = w[1];
      }
#pragma unroll
      for (int nt = 0; nt < 2; ++nt)
        o[dt][nt] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(vf, pf.f8[nt], o[dt][nt], 0, 0, 0, 127, 0, 127);
    } else {
      LDS v4s_t* base = lds_at<v4s_t>(v_lane + ((dt ^ jj) << 5));
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const v2u_t w0 = __builtin_bit_cast(v2u_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16(base + (32 * u) * 32));  // (32u) rows * 256 B
        const v2u_t w1 = __builtin_bit_cast(v2u_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16(base + (32 * u + 16) * 32));
        const v8bf vf = __builtin_bit_cast(v8bf, make_uint4(w0[0], w0[1], w1[0], w1[1]));
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
          const uint4 w = make_uint4(pf.b16w[u][nt][0], pf.b16w[u][nt][1], pf.b16w[u][nt][2], pf.b16w[u][nt][3]);
          o[dt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, __builtin_bit_cast(v8bf, w), o[dt][nt], 0, 0, 0);
        }
      }
    }
  }

  __device__ __forceinline__ uint32_t v_lane_addr(int buf) const {
    const uint32_t vt = lds_base + L::OFF_V + buf * L::V_BYTES;
    const int jj = FP8V ? (n16 >> 1) : (n16 >> 2);
    return FP8V ? vt + (16 * (jj >> 2) + 4 * g + (jj & 3)) * 128 + 8 * (n16 & 1)
                : vt + (4 * g + jj) * 256 + 8 * (n16 & 1) + 16 * ((n16 & 3) >> 1);
  }

  // o_sum += 1^T P^T: the rounded probabilities summed on the matrix core with an all-ones
  // V^T tile, so O can be normalised by exactly the weights it was accumulated with.
  // Only the BF16 mode needs it: there the probabilities are taken against a stale maximum.
  __device__ __forceinline__ void pv_sum(const PFrag& pf) {
    if (!FP8V) {
      const v8bf ones = __builtin_bit_cast(v8bf, make_uint4(0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u));
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
          const uint4 w = make_uint4(pf.b16w[u][nt][0], pf.b16w[u][nt][1], pf.b16w[u][nt][2], pf.b16w[u][nt][3]);
          o_sum[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, __builtin_bit_cast(v8bf, w), o_sum[nt], 0, 0, 0);
        }
    }
  }

  // P V of a whole block resident in V buffer `buf`.
  __device__ __forceinline__ void pv(int buf, const PFrag& pf) {
    const uint32_t v_lane = v_lane_addr(buf);
    const int jj = FP8V ? (n16 >> 1) : (n16 >> 2);
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) pv_tile(v_lane, dt, jj, pf);
    pv_sum(pf);
  }

  __device__ __forceinline__ void rescale(const float alpha[2]) {
#pragma unroll
    for (int dt = 0; dt < 8; ++dt)
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) o[dt][nt] *= alpha[nt];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) o_sum[nt] *= alpha[nt];
  }

  // ---------------------------------------------------------------- one pipeline iteration
  // Softmax of block j (scores in s -> P(j) in pf_cur), scores of block j+1 written back into
  // s (if DO_QK) and O += P(j-1) V(j-1) (if DO_PV). Issued as 8 slots: slot k turns score tile k
  // into probabilities, then overwrites it with the next block's score tile k, and runs the
  // P V instructions of d tile k, so matrix and vector work overlap and live ranges stay short.
  template <bool DO_QK, bool DO_PV, bool MASK>
  __device__ __forceinline__ void step(int j, v4f s[8][2], const PFrag& pf_prev, PFrag& pf_cur) {
    if (MASK) {
      const int kb = j * BN;
#pragma unroll
      for (int mt = 0; mt < 8; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (kb + 16 * mt + 4 * g + i >= Lk) {
            s[mt][0][i] = -INFINITY;
            s[mt][1][i] = -INFINITY;
          }
    }
    // Row maxima of block j. The running maximum m_run is only moved when some row of the wave
    // exceeds it by more than Lazy<FP8V>::LOG2; otherwise probabilities are taken against the
    // stale maximum (they stay <= 2^LOG2, well inside BF16 range) and O needs no rescale.
    float rs[2] = {0.0f, 0.0f};
    bool move = false;
    float cand[2];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      float mx = -INFINITY;
#pragma unroll
      for (int mt = 0; mt < 8; ++mt)
        mx = fmaxf(fmaxf(mx, fmaxf(s[mt][nt][0], s[mt][nt][1])), fmaxf(s[mt][nt][2], s[mt][nt][3]));
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      cand[nt] = mx * c;
      move = move || (cand[nt] > m_run[nt] + Lazy<FP8V>::LOG2);
    }
    // O still lacks P(j-1) V(j-1), which was taken against the old maximum: O is rescaled after
    // that product has been added (end of this step); l has no such lag.
    const bool moved = __ballot(move) != 0;  // wave-uniform, rare after the first block
    const bool first = m_run[0] == -INFINITY;  // same for every lane: nothing accumulated yet
    float alpha[2] = {1.0f, 1.0f};
    if (moved) {
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        const float m_new = fmaxf(m_run[nt], cand[nt]);
        alpha[nt] = __builtin_amdgcn_exp2f(m_run[nt] - m_new);
        l_run[nt] *= alpha[nt];
        m_run[nt] = m_new;
      }
    }
    const float m_use[2] = {m_run[0], m_run[1]};

    const uint32_t kt = lds_base + L::OFF_K + ((j + 1) & 1) * L::K_BYTES;
    LDS const uint32_t* ksc = lds_at<const uint32_t>(lds_base + L::OFF_KSC + ((j + 1) & 1) * L::KSC_BYTES);
    LDS const v4u_t* k_a = lds_at<const v4u_t>(kt + n16 * 128 + ((g ^ (n16 & 7)) << 4));
    LDS const v4u_t* k_b = lds_at<const v4u_t>(kt + n16 * 128 + (((4 + g) ^ (n16 & 7)) << 4));
    const uint32_t v_lane = v_lane_addr((j + 2) % 3);   // V(j-1)
    const int jj = FP8V ? (n16 >> 1) : (n16 >> 2);

#pragma unroll
    for (int k = 0; k < 8; ++k) {
      // probabilities of score tile k of block j
#pragma unroll
      for (int nt = 0; nt < 2; ++nt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float pv = __builtin_amdgcn_exp2f(fmaf(s[k][nt][i], c, -m_use[nt]));
          s[k][nt][i] = pv;
          rs[nt] += pv;
        }
      if (FP8V) {
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
          pf_cur.f8[nt][k] = (int)cvt4_e4m3(s[k][nt][0], s[k][nt][1], s[k][nt][2], s[k][nt][3]);
      } else {
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
          pf_cur.b16w[k >> 1][nt][2 * (k & 1)] = cvt_pk_bf16(s[k][nt][0], s[k][nt][1]);
          pf_cur.b16w[k >> 1][nt][2 * (k & 1) + 1] = cvt_pk_bf16(s[k][nt][2], s[k][nt][3]);
        }
      }
      if (DO_QK) {  // scores of block j+1, key tile k (overwrites the consumed tile)
        const v8i kf = make_v8i(k_a[k * 128], k_b[k * 128]);            // + k * 2048 bytes
        const int ks = MX ? (int)((ksc[16 * k + n16] >> (8 * g)) & 0xFFu) : 127;
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
          s[k][nt] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(kf, qf[nt], v4f{0.0f, 0.0f, 0.0f, 0.0f},
                                                                      0, 0, 0, ks, 0, qsc[nt]);
      }
      if (DO_PV) {
        pv_tile(v_lane, k, jj, pf_prev);
        if (k == 7) pv_sum(pf_prev);
      }
      __builtin_amdgcn_sched_barrier(0);  // keep slot k's operand loads from being hoisted further
    }
    l_run[0] += rs[0];
    l_run[1] += rs[1];
    if (moved && !first) rescale(alpha);
  }

  // Iteration j: loads K(j+2) into K buffer j%2 and V(j+1) into V buffer (j+1)%3, the pipelined
  // step (scores of block j+1 on the FP8 path when FAST, else by the BF16 path after the step),
  // then waits for this iteration's loads and synchronises the workgroup.
  template <bool FAST, bool FIRST, bool LAST>
  __device__ __forceinline__ void iteration(int j, v4f s[8][2], PFrag& pf_prev, PFrag& pf_cur) {
    if (j + 2 < nb) dma_k(j + 2, j & 1);
    if (!LAST) dma_v(j + 1, (j + 1) % 3);
    step<FAST && !LAST, !FIRST, LAST>(j, s, pf_prev, pf_cur);
    if (!FAST && !LAST) scores_bf16((j + 1) & 1, s);
    pf_prev = pf_cur;
    wait_vm_all();
    __syncthreads();
  }

  template <bool FAST>
  __device__ __forceinline__ void main_loop() {
    v4f s[8][2];
    PFrag pf_prev, pf_cur;
    if (FAST) scores_fp8(0, s); else scores_bf16(0, s);
    __syncthreads();  // K buffer 0 is reused for block 2
    if (nb == 1) {
      iteration<FAST, true, true>(0, s, pf_prev, pf_cur);
    } else {
      iteration<FAST, true, false>(0, s, pf_prev, pf_cur);
      for (int j = 1; j < nb - 1; ++j) iteration<FAST, false, false>(j, s, pf_prev, pf_cur);
      iteration<FAST, false, true>(nb - 1, s, pf_prev, pf_cur);
    }
    pv((nb - 1) % 3, pf_prev);   // the last block's P V (pf_prev holds P(nb-1) now)
  }

  __device__ __forceinline__ void run(int qtile) {
    H = p.num_heads;
    const int q_start = p.cu_q[seq];
    const int Lq = p.cu_q[seq + 1] - q_start;
    const int q0 = qtile * BM;
    const int k_start = p.cu_k[seq];
    Lk = p.cu_k[seq + 1] - k_start;
    nb = (Lk + BN - 1) / BN;
    const int tid = threadIdx.x;
    lane = tid & 63;
    wave = tid >> 6;
    n16 = lane & 15;
    g = lane >> 4;

    const float qd = p.q_descale ? p.q_descale[seq * p.qd_ss + head * p.qd_sh] : 1.0f;
    const float kd = p.k_descale ? p.k_descale[seq * p.kd_ss + head * p.kd_sh] : 1.0f;
    c = (p.scale_log2 * qd) * kd;  // identical arithmetic with or without descales

    kbase = p.k + (int64_t)k_start * p.k_st + (int64_t)head * p.k_sh;
    vbase = reinterpret_cast<const uint8_t*>(p.v) + ((int64_t)k_start * p.v_st + (int64_t)head * p.v_sh) * (FP8V ? 1 : 2);
    k_st_b = p.k_st;
    v_st_b = p.v_st * (FP8V ? 1 : 2);
    ksc_base = MX ? p.k_scale + ((int64_t)p.cu_scale_k[seq] * H + head) * 4 : nullptr;

    // start the first loads before touching Q
    if (nb > 0) {
      dma_k(0, 0);
      dma_v(0, 0);
      if (nb > 1) dma_k(1, 1);
    }

    // ---- Q fragments: FP8 (score B operand) and exactly dequantized BF16 (guarded path) ----
    uint32_t qmax_code = 0, qmax_scale = 0;
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      const int qi = q0 + wave * 32 + nt * 16 + n16;
      if (qi < Lq) {
        const uint8_t* qp = p.q + (int64_t)(q_start + qi) * p.q_st + (int64_t)head * p.q_sh;
        const uint4 a = ldg16(qp + 16 * g), b = ldg16(qp + 64 + 16 * g);
        qf[nt] = make_v8i(a, b);
        const uint32_t sw = MX ? *reinterpret_cast<const uint32_t*>(p.q_scale + (((int64_t)p.cu_scale_q[seq] + qi) * H + head) * 4)
                               : 0x7F7F7F7Fu;
        qsc[nt] = (int)((sw >> (8 * g)) & 0xFFu);
        qrow[nt] = qp;
        qsw[nt] = sw;
        uint32_t words[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const uint32_t w = words[i] & 0x7F7F7F7Fu;
          qmax_code = max(qmax_code, max(max(w & 0xFF, (w >> 8) & 0xFF), max((w >> 16) & 0xFF, w >> 24)));
        }
        qmax_scale = max(qmax_scale, (uint32_t)qsc[nt]);
      } else {
        qf[nt] = make_v8i(make_uint4(0, 0, 0, 0), make_uint4(0, 0, 0, 0));
        qsc[nt] = 127;
        qrow[nt] = nullptr;
        qsw[nt] = 0x7F7F7F7Fu;
      }
    }
    if (MX) {
      qbound = 448.0f * e8m0_to_float(wave_max_u32(qmax_scale));
    } else {
      // largest E4M3 magnitude among the wave's query codes (codes order like magnitudes)
      const uint32_t mc = wave_max_u32(qmax_code);
      qbound = __builtin_amdgcn_cvt_f32_fp8((int)mc, 0);
    }

    m_run[0] = m_run[1] = -INFINITY;
    l_run[0] = l_run[1] = 0.0f;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt)
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) o[dt][nt] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
    o_sum[0] = o_sum[1] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

    if (nb > 0) {
      const bool fast = fp8_scores_ok_tile(reinterpret_cast<float*>(lds + L::TOTAL - 16));
      wait_vm_all();
      __syncthreads();
      if (fast) main_loop<true>(); else main_loop<false>();
    }

    // ---- epilogue: O = O^T / l * vd -> BF16; LSE = ln2 * (m + log2 l) ----
    const float vd = p.v_descale ? p.v_descale[seq * p.vd_ss + head * p.vd_sh] : 1.0f;
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      float lt = l_run[nt] + __shfl_xor(l_run[nt], 16);
      lt += __shfl_xor(lt, 32);
      const int qi = q0 + wave * 32 + nt * 16 + n16;
      if (qi < Lq) {
        // BF16 mode: the sum of the rounded probabilities (every row of the ones tile holds it);
        // FP8 mode: the FP32 sum (the largest probability is exactly 1 there).
        const float ls = FP8V ? lt : o_sum[nt][0];
        const float inv = ls > 0.0f ? 1.0f / ls : 0.0f;
        uint16_t* op = p.out + ((int64_t)(q_start + qi) * H + head) * 128 + 4 * g;
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) {
          const v4f x = o[dt][nt];
          const uint2 w = make_uint2(cvt_pk_bf16((x[0] * inv) * vd, (x[1] * inv) * vd),
                                     cvt_pk_bf16((x[2] * inv) * vd, (x[3] * inv) * vd));
          *reinterpret_cast<uint2*>(op + 16 * dt) = w;
        }
        if (g == 0)
          p.lse[(int64_t)head * p.total_q + q_start + qi] =
              lt > 0.0f ? (m_run[nt] + __builtin_amdgcn_logf(lt)) * LN2 : -INFINITY;
      }
    }
  }
};

template <bool MX, bool FP8V>
__global__ __launch_bounds__(256) void attn_fwd_kernel(AttnParams p) {
  extern __shared__ __align__(16) uint8_t smem[];
  int seq, head, qtile;
  if (p.tile_order != nullptr) {
    if ((int)blockIdx.x >= p.num_tiles) return;
    seq = p.tile_order[3 * blockIdx.x];
    head = p.tile_order[3 * blockIdx.x + 1];
    qtile = p.tile_order[3 * blockIdx.x + 2];
  } else {
    const int per_xcd = (int)(gridDim.x >> 3);  // grid is a multiple of 8
    const int logical = (int)(blockIdx.x & 7) * per_xcd + (int)(blockIdx.x >> 3);
    if (logical >= p.num_tiles) return;
    qtile = logical % p.q_tiles;
    const int rest = logical / p.q_tiles;
    head = rest % p.num_heads;
    seq = rest / p.num_heads;
  }
  if (qtile * BM >= p.cu_q[seq + 1] - p.cu_q[seq]) return;
  Attn<MX, FP8V> a(p, smem);
  a.seq = seq;
  a.head = head;
  a.run(qtile);
}

template <bool MX, bool FP8V>
hipError_t launch_variant(const AttnParams& p, dim3 grid, hipStream_t s, hipEvent_t start, hipEvent_t stop) {
  // Raising the dynamic LDS limit is a per-kernel, per-device attribute: done once per device.
  static std::atomic<uint64_t> configured{0};
  const int bytes = Lay<FP8V>::TOTAL;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const uint64_t bit = dev < 64 ? (uint64_t(1) << dev) : 0;
  if (bit == 0 || !(configured.load(std::memory_order_acquire) & bit)) {
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(&attn_fwd_kernel<MX, FP8V>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
    if (e != hipSuccess) return e;
    configured.fetch_or(bit, std::memory_order_acq_rel);
  }
  if (start == nullptr && stop == nullptr) {
    hipLaunchKernelGGL((attn_fwd_kernel<MX, FP8V>), grid, dim3(256), bytes, s, p);
    return hipGetLastError();
  }
  // The dispatch itself stamps the events: their interval is the kernel, without launch gaps.
  AttnParams arg = p;
  void* args[] = {&arg};
  return hipExtLaunchKernel(reinterpret_cast<const void*>(&attn_fwd_kernel<MX, FP8V>), grid, dim3(256), args,
                            bytes, s, start, stop, 0);
}

}  // namespace

hipError_t launch_attention(const AttnParams& p, bool mx, int pv_mode, hipStream_t s, hipEvent_t start,
                            hipEvent_t stop) {
  if (p.num_tiles == 0) {
    if (start) {
      hipError_t e = hipEventRecord(start, s);
      if (e != hipSuccess) return e;
    }
    return stop ? hipEventRecord(stop, s) : hipSuccess;
  }
  unsigned grid = (unsigned)p.num_tiles;
  if (p.tile_order == nullptr) grid = (grid + 7u) & ~7u;  // XCD remap needs a multiple of 8
  const bool fp8v = pv_mode == LPFA_PV_FP8;
  if (mx && fp8v) return launch_variant<true, true>(p, dim3(grid), s, start, stop);
  if (mx) return launch_variant<true, false>(p, dim3(grid), s, start, stop);
  if (fp8v) return launch_variant<false, true>(p, dim3(grid), s, start, stop);
  return launch_variant<false, false>(p, dim3(grid), s, start, stop);
}

}  // namespace lpfa
