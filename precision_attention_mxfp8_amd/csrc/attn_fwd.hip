// Fused noncausal head_dim-128 attention forward over packed sequences, gfx950 (CDNA4).
//
// What is computed: LP-FA4 README (introduction; section "MXFP8 forward and backward"):
// MXFP8 Q/K, noncausal MHA, (out, lse); FastVideo fp8-PV PR: V is BF16 or an unscaled E4M3
// cast read with dequant scale 1.0, output BF16; vLLM unit-descale PR: optional per-tensor
// descales, a missing one read as 1.0 through the same arithmetic.
//
// Work split: one workgroup = one (sequence, head, 128-query tile). A wave group is 4 waves x
// 32 queries. With E4M3 V the workgroup has two wave groups that take alternate 128-key
// blocks (group 0 the even ones, group 1 the odd ones) and merge their partial (m, l, O) at
// the end; each SIMD then holds two waves, so the matrix work and waits of one overlap the
// softmax of the other. BF16 V tiles are twice as large: one group (LDS would not hold two).
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
//    The per-lane part of every load address is fixed for the whole sequence; each block only
//    moves a uniform base. Only a sequence's last, partial block clamps rows to the last key.
//  * Each group double-buffers K and V: in its local iteration j it loads K for its block j+2
//    and V for its block j, and waits for both at the end of the iteration.
//
// Pipeline (local iteration j): the score instructions for block j+1 and the P V instructions
// for block j-1 overlap the softmax VALU work of block j. The running maximum is lazy: it only
// moves when a row's maximum exceeds it by more than 2^8, so the probabilities stay <= 256
// (inside E4M3 and BF16 range) and O is rarely rescaled. O is normalised by the sum of the
// probabilities as rounded for the P V instruction (summed on the matrix core against an
// all-ones tile), so a dominant probability's rounding cancels; LSE uses the unrounded FP32
// sum. The loop is unrolled twice so that the probability fragments of consecutive blocks
// alternate between two register sets without copies.
//
// Precision guard: the FP8 matrix instructions do not accumulate exactly. Inside each group of 8
// consecutive products every product is truncated toward zero onto the grid 2^(E - 13), E being
// the group's largest exponent sum (exponent of q plus exponent of k); the group sums then
// accumulate in FP32. Seven products per group can each lose almost one grid step, so a score's
// error is below 7 * 2^-13 * sum over the 16 groups of 2^E (times the block scales), i.e. at
// most about 2^-6.2 * max|q| * max|k| in magnitude. Random-sign data loses little (the
// truncations cancel); same-sign products spanning more than 2^7 inside a group lose the most.
// Before the key loop the workgroup bounds c * max|q| * max|k| (c = softmax_scale * log2 e *
// descales; in MX mode from the E8M0 scales: block maxima lie in (224, 448] * 2^e; in
// per-tensor mode from the E4M3 codes of Q, and for K from the per-16-row code maxima that the
// cast writes, or the E4M3 range 448 without them). Above the threshold (16 by default: scores
// then err by at most ~0.22 in log2 units, typically by ~1e-4 on N(0,1) data) the scores are
// computed instead with v_mfma_f32_16x16x32_bf16 on exactly dequantized operands
// (v_cvt_scalef32_pk_bf16_fp8), whose FP32 accumulation of exact BF16 products loses nothing
// here. Typical N(0,1) data stays on the FP8 path; tiles whose rows meet outliers take the BF16
// path.
//
// Workgroup ids are remapped so that all tiles of one (sequence, head) land on the same XCD (ids
// are dealt round-robin over the 8 XCDs), sharing K/V in that XCD's L2; with a head count that is
// a multiple of 8, head h goes to XCD h % 8, where the preparation kernels wrote its codes.
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
// Stale-maximum slack of the online softmax, in log2 units: probabilities may be taken against
// a maximum up to 8 below the running one (P <= 2^8).
constexpr float LAZY_LOG2 = 8.0f;
// Two-group softmax: largest sum of one lane's probabilities of a row taken against a stale
// maximum (it bounds each of them, as LAZY_LOG2 does for the one-group kernel)
constexpr float LAZY_SUM = 256.0f;

template <bool FP8V>
struct Groups { static constexpr int G = FP8V ? 2 : 1; };

template <bool FP8V, bool QB = false>
struct Lay {
  static constexpr int K_BYTES = BN * (QB ? 256 : 128);  // QB: BF16 keys (256-byte rows)
  static constexpr int KSC_BYTES = BN * 4;
  static constexpr int V_BYTES = FP8V ? BN * 128 : BN * 256;
  // Dynamic LDS: K and its scales (read with ordinary LDS loads).
  static constexpr int OFF_K = 0;                        // 2 buffers
  static constexpr int OFF_KSC = 2 * K_BYTES;            // 2 buffers
  // V's token-block scales (MX V): per buffer 4 rows (32-key quarters) of 128 bytes (d)
  static constexpr int VSC_BYTES = 4 * 128;
  static constexpr int OFF_VSC = OFF_KSC + 2 * KSC_BYTES;  // 2 buffers (E4M3 V only)
  static constexpr int GROUP_BYTES = OFF_VSC + (FP8V ? 2 * VSC_BYTES : 0);
  static constexpr int OFF_RED = Groups<FP8V>::G * GROUP_BYTES;  // guard reduction slots
  // Q fragments (score B operands) of the 4 query waves: per (wave, 16-query tile) two 1 KB
  // halves, lane L's 16-byte pieces at L * 16 (conflict-free 16-byte reads). Reloaded for
  // each score phase instead of held in registers.
  static constexpr int OFF_Q = OFF_RED + 64;
  static constexpr int TOTAL = OFF_Q + 4 * 2 * 2048;
  // V buffers live in two static LDS objects of 32 KB, apart from the dynamic K area, so loads
  // in flight into K never hold up the transposing V reads (the compiler makes those reads wait
  // for every outstanding load into the same object). One group: object i is V buffer i. Two
  // groups: object g holds group g's two V buffers, and each group issues its V loads only
  // after its own V reads of the iteration. The merge of the two groups passes half of each
  // group's O (8 v4f per lane per wave) through the group's K buffers and its (m, l, rounded
  // sum) (2 v4f per lane per wave) through half of the Q area.
  static constexpr int VOBJ_BYTES = 32768;
  static_assert(V_BYTES * Groups<FP8V>::G == VOBJ_BYTES, "V objects");
  static_assert(Groups<FP8V>::G == 1 || (4 * 8 * 64 * 16 <= 2 * K_BYTES && 2 * 4 * 2 * 64 * 16 <= 4 * 2 * 2048), "merge area");
};

typedef int v2i_t __attribute__((ext_vector_type(2)));
typedef short v4s_t __attribute__((ext_vector_type(4)));
typedef unsigned v2u_t __attribute__((ext_vector_type(2)));
typedef unsigned v4u_t __attribute__((ext_vector_type(4)));
// BF16 operands are always assembled from whole 32-bit words: building them element by element
// from 16-bit values lets the compiler repack halves (it has emitted a repack that dropped the
// second register of a transposed read).
#define LDS __attribute__((address_space(3)))
#define LDS_PTR(T, p) ((LDS T*)(p))
// LDS byte address (32-bit) -> typed LDS pointer, so offsets fold into the DS immediate field.
template <typename T>
__device__ __forceinline__ LDS T* lds_at(uint32_t byte_addr) {
  return reinterpret_cast<LDS T*>(static_cast<uintptr_t>(byte_addr));
}

__device__ __forceinline__ uint4 ldg16(const void* p) { return *reinterpret_cast<const uint4*>(p); }
__device__ __forceinline__ uint2 ldg8(const void* p) { return *reinterpret_cast<const uint2*>(p); }

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

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t x) {
#pragma unroll
  for (int s = 1; s < 64; s <<= 1) x = max(x, (uint32_t)__shfl_xor((int)x, s));
  return x;
}

// max over lanes i, i^16, i^32, i^48 (the 4 lane groups holding one query row) with the
// gfx950 lane-swap instructions: with both operands equal, the 16-swap pairs row r with r^1 and
// the 32-swap pairs the two halves.
__device__ __forceinline__ float xmax16_32(float x) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// Ends a scheduling region: no instruction is moved across it, and (compiler-only memory
// fence, no instruction emitted) no memory access either, so LDS operand reads stay with
// the matrix instructions that use them instead of all being hoisted ahead.
__device__ __forceinline__ void region_end() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("" ::: "memory");
}

__device__ __forceinline__ void wait_vm_all() { __builtin_amdgcn_s_waitcnt(0x0F70); }  // vmcnt(0)

// Probability fragments of one key block (B operand of the P V instructions).
//   fp8 mode:  one v8i per 16-query tile; byte 4*mt + i = key 16*mt + 4*g + i.
//   bf16 mode: per 32-key chunk u and query tile, 4 words; element j = key 32u + 16*(j/4) + 4*g + j%4.
template <bool FP8V>
struct PFrag;
template <>
struct PFrag<true> { v8i f8[2]; };
template <>
struct PFrag<false> { uint32_t w[4][2][4]; };

// MX: Q and K carry E8M0 block scales. FP8V: V is E4M3 (two wave groups). VMX: that E4M3 V
// carries E8M0 scales per 32 tokens (the P V instruction's A-operand scales). DQ: the guarded
// path of the BF16-V kernel: MX Q and K dequantized exactly to BF16 (Q once per tile into
// registers, K once per block into BF16 LDS tiles), then the BF16 pipeline below. QB: Q and K are
// BF16 (the BF16 FlashAttention forward: BF16 scores and BF16 P V, one wave group).
template <bool MX, bool FP8V, bool VMX, bool QB = false, bool DQ = false, bool DQS = false>
struct Attn {
  static_assert(!QB || (!MX && !FP8V && !VMX), "BF16 Q/K come with BF16 V only");
  static_assert(!DQ || (MX && !FP8V && !VMX && !QB), "the dequantized path is the BF16-V kernel's");
  static_assert(!DQS || DQ, "K's BF16 values from the quantizer serve the DQ pipeline");
  static constexpr bool KB16 = QB || DQ;  // K in LDS and Q in registers are BF16
  using L = Lay<FP8V, KB16>;
  using PF = PFrag<FP8V>;
  static constexpr int G = Groups<FP8V>::G;
  static constexpr bool QREG = G == 2;  // FP8 Q fragments in registers (q_frags)

  // ---- per-workgroup constants ----
  const AttnParams& p;
  uint8_t* lds;              // this wave group's K buffers (dynamic LDS)
  uint32_t lds_base;         // the same, as an LDS byte address
  LDS uint8_t* vobj[2];      // the two static V objects; always indexed by constants
  int seq, head, H, Lk, nb;
  int q_start, Lq, k_start;  // the sequence's first query and key rows, and its query count
  int qtile0;                // this tile's index among the sequence's query tiles
  int scq, sck;              // its first scale rows (MX mode)
  int lane, wave, n16, g;    // wave: index inside the group (queries 32*wave ..)
  int grp, ng;               // wave group, and the number of key blocks it processes
  const uint8_t* kbase;      // key row 0 of this (sequence, head) (DQS: of K's BF16 values)
  const uint8_t* kend;       // one past the last byte of that tensor
  const uint8_t* vbase;      // value row 0 (bytes)
  int64_t k_st_b, v_st_b;    // row strides in bytes
  const uint8_t* ksc_base;   // scale word of key row 0 of this (sequence, head)
  const uint8_t* kgm_base;   // the guard's K maxima of this (sequence, head), if given (see guard_count)
  int gcount;                // elements of the guard's K data
  float c;                   // softmax_scale * log2(e) * qd * kd


  // ---- per-wave state ----
  int qsc[2];
  v8i qreg[2];  // two-group kernel: this wave's FP8 Q fragments, held in registers
  v8bf qb16[2][4];           // QB, DQ: Q fragments, query tile nt, head_dim slice 32u .. 32u + 31
  uint4 kpre[4];             // DQ: this lane's staged K chunks of the next block (FP8), and
  uint32_t kpre_sc[4];       // their rows' scale words
  float qbound;              // max |q| bound of the wave's queries
  uint32_t ksw[8];           // first batch of the guard's K scale words, loaded before Q
  const uint8_t* qrow[2];    // this lane's query rows (nullptr past the end)
  uint32_t qsw[2];           // their E8M0 scale words
  float m_run[2], l_run[2];
  v4f o[8][2];
  v4f o_sum[2];              // sum over keys of the rounded probabilities (ones tile of V^T)

  __device__ Attn(const AttnParams& p_, uint8_t* lds_, int grp_, LDS uint8_t* va, LDS uint8_t* vb)
      : p(p_), lds(lds_ + grp_ * L::GROUP_BYTES),
        lds_base((uint32_t)(uintptr_t)(LDS uint8_t*)lds_ + grp_ * L::GROUP_BYTES), grp(grp_) {
    vobj[0] = va;
    vobj[1] = vb;
  }

  // key block processed by this group in its local iteration i
  __device__ __forceinline__ int blk(int i) const { return G * i + grp; }

  // One group: its LDS reads are addressed as a single opaque per-lane offset from their object
  // (V object or dynamic area), so that the compiler can tell which object each read touches
  // (it follows only a few address steps back to the object, and otherwise waits for every load
  // into LDS in flight). The empty asm emits nothing; it only keeps the offset in one piece.
  __device__ __forceinline__ static uint32_t opaque(uint32_t x) {
    asm("" : "+v"(x));
    return x;
  }
  __device__ __forceinline__ LDS uint8_t* dyn() const { return LDS_PTR(uint8_t, lds); }

  // ---------------------------------------------------------------- global -> LDS
  // Buffer loads straight to LDS: the block's base (uniform) goes into a buffer descriptor
  // whose range ends at the tensor's last byte, so rows past the end of the last sequence
  // read zeros (rows past a sequence's end inside the tensor are other sequences' keys: masked
  // scores, zero probabilities). Each lane's 32-bit offsets are fixed for the whole sequence.
  // K: instruction i of wave w fills 1 KB region R = 4w + i = LDS rows 8R..8R+7; lane L fills
  // row 8R + L/8 with chunk (L%8) ^ (L/8) of its key. V fp8: same rows, chunk (L%8) ^ ((L/8)%4 |
  // 4*(i/2)). With E4M3 V the LDS rows hold the keys in the permuted order below (perm_base),
  // else LDS row = key. V bf16: region R = 8w + i = rows 4R..4R+3 of 256 B; lane L fetches row
  // 4R + L/16, chunk (L%16) ^ 2((L/16)%4).
  // K scales: waves 0 and 1 fetch 64 rows each, one 4-byte word per lane (the scale storage is
  // padded to whole blocks, so every row exists).
  // The row step between a wave's instructions goes into the (uniform) instruction offset; each
  // lane's offset is recomputed from its lane id at load time (a few integer instructions)
  // rather than held in registers across the loop.
  __device__ __forceinline__ uint32_t k_off() const {
    const int r8 = lane >> 3;
    return (uint32_t)(r8 * (int)k_st_b) + 16u * ((lane & 7) ^ r8);
  }
  __device__ __forceinline__ uint32_t v_off(int) const {  // BF16 V
    const int r4 = lane >> 4;
    return (uint32_t)(r4 * (int)v_st_b) + 16u * ((lane & 15) ^ (2 * (r4 & 3)));
  }

  // Buffer descriptor for [base, end): raw (stride 0), range = remaining bytes (clamped).
  __device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const uint8_t* base, const uint8_t* end) const {
    const int64_t left = end - base;
    const int n = left <= 0 ? 0 : (left >= 0x7FFFFFFF ? 0x7FFFFFFF : (int)left);
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(base), (short)0, n, 0x00020000);
  }

  // Key order in LDS for E4M3 V. P (the P V instruction's B operand, as the scores left it)
  // holds in dword t, byte i of lane group g the key of LDS row 16t + 4g + i, and V's
  // transposed reads follow the LDS rows the same way. The 16x16x128 FP8 instruction takes
  // K slots 16g + 4t + i (t < 4) and 64 + 16g + 4(t - 4) + i (t >= 4) from those places, and
  // applies scale block b to slots 32b .. 32b + 31. LDS row 16t + 4g + i therefore holds key
  // 64(t/4) + 16g + 4(t%4) + i: slot s then carries key s, and with V in MXFP8 along tokens
  // scale block b is exactly V's 32-token block b of the key block. For the rows one lane fills
  // (LDS rows 32w + 8i + r, r = lane / 8, instruction i of wave w) the key is
  // perm_base(r) + perm_step(i): a lane part and a uniform per-instruction part.
  __device__ __forceinline__ int perm_base(int r) const {
    return 16 * (r >> 2) + (r & 3) + 64 * (wave >> 1) + 8 * (wave & 1);
  }
  __device__ __forceinline__ static int perm_step(int i) { return 32 * (i & 1) + 4 * (i >> 1); }

  // K block b into K buffer buf of wave group tg (the issuing wave's group may differ; tg is a
  // constant at every call).
  __device__ __forceinline__ void dma_k(int tg, int b, int buf) {
    uint8_t* area = lds + (tg - grp) * L::GROUP_BYTES;
    LDS uint8_t* dst = LDS_PTR(uint8_t, area + L::OFF_K + buf * L::K_BYTES + 4 * wave * 1024);
    if constexpr (QB || DQS) {
      // BF16 rows of 256 bytes: instruction i of wave w fills region 8w + i = rows 32w + 4i ..
      // 32w + 4i + 3; lane L fills row 32w + 4i + L/16, LDS chunk L%16, with the row's chunk
      // (L%16) ^ (row%16) (the score reads then hit 16 different banks for 16 rows)
      LDS uint8_t* qdst = LDS_PTR(uint8_t, area + L::OFF_K + buf * L::K_BYTES + 8 * wave * 1024);
      const int r16 = lane >> 4;
      const auto r = rsrc(kbase + (int64_t)(b * BN + 32 * wave) * k_st_b, kend);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int row = 4 * i + r16;  // (32w + row) % 16 == row % 16
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (LDS void*)(qdst + i * 1024), 16,
                                                 (uint32_t)(row * (int)k_st_b) + 16u * ((lane & 15) ^ (row & 15)),
                                                 0, 0, 0);
      }
    } else if constexpr (FP8V) {
      const int r8 = lane >> 3;
      const uint32_t off = (uint32_t)(perm_base(r8) * (int)k_st_b) + 16u * ((lane & 7) ^ r8);
      const auto r = rsrc(kbase + (int64_t)(b * BN) * k_st_b, p.k_end);
#pragma unroll
      for (int i = 0; i < 4; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (LDS void*)(dst + i * 1024), 16,
                                                 off + (uint32_t)perm_step(i) * (uint32_t)k_st_b, 0, 0, 0);
    } else {
      const uint8_t* row0 = kbase + (int64_t)(b * BN + 32 * wave) * k_st_b;
      const uint32_t off = k_off();
      const auto r = rsrc(row0, p.k_end);  // one descriptor per block; the row step goes into the offsets
#pragma unroll
      for (int i = 0; i < 4; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (LDS void*)(dst + i * 1024), 16,
                                                 off + (uint32_t)(8 * i) * (uint32_t)k_st_b, 0, 0, 0);
    }
    if (MX && wave < 2) {
      // scale words of LDS rows 64w + L (w = 0, 1): key 64w + 16((L/4)%4) + 4(L/16) + L%4 with E4M3 V
      const int krow = FP8V ? 64 * wave + 16 * ((lane >> 2) & 3) + 4 * (lane >> 4) + (lane & 3) : 64 * wave + lane;
      const auto rs = rsrc(ksc_base + (int64_t)(b * BN) * H * 4, ksc_base + (int64_t)(b * BN + BN) * H * 4);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (LDS void*)(area + L::OFF_KSC + buf * L::KSC_BYTES + wave * 256), 4,
                                               (uint32_t)(krow * H * 4), 0, 0, 0);
    }
  }

  // V block b into V buffer y of static object obj (a constant at every call).
  __device__ __forceinline__ void dma_v(int obj, int b, int y) {
    constexpr int N = FP8V ? 4 : 8;              // 1 KB regions per wave
    constexpr int ROWS = FP8V ? 8 : 4;           // key rows per region
    LDS uint8_t* dst = (obj == 0 ? vobj[0] : vobj[1]) + y * L::V_BYTES + N * wave * 1024;
    if constexpr (FP8V) {  // rows in the permuted key order of dma_k
      const int r8 = lane >> 3;
      const uint32_t base = (uint32_t)(perm_base(r8) * (int)v_st_b);
      const uint32_t off0 = base + 16u * ((lane & 7) ^ (r8 & 3)), off1 = base + 16u * ((lane & 7) ^ ((r8 & 3) | 4));
      const auto r = rsrc(vbase + (int64_t)(b * BN) * v_st_b, p.v_end);
#pragma unroll
      for (int i = 0; i < N; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (LDS void*)(dst + i * 1024), 16,
                                                 ((i & 2) ? off1 : off0) + (uint32_t)perm_step(i) * (uint32_t)v_st_b, 0, 0, 0);
      if (VMX && wave < 2) {  // the block's 4 scale rows (32-key quarters), 2 per wave
        const uint8_t* sb = p.v_scale + (((int64_t)sck / 32 + 4 * b + 2 * wave) * H + head) * 128;
        const auto rs = rsrc(sb, sb + (int64_t)H * 128 + 128);
        LDS uint8_t* sd = LDS_PTR(uint8_t, lds + (obj - grp) * L::GROUP_BYTES + L::OFF_VSC + y * L::VSC_BYTES + wave * 256);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (LDS void*)sd, 4, (uint32_t)((lane >> 5) * H * 128 + (lane & 31) * 4),
                                                 0, 0, 0);
      }
    } else {
      const uint8_t* row0 = vbase + (int64_t)(b * BN + N * ROWS * wave) * v_st_b;
      const uint32_t off0 = v_off(0);
      const auto r = rsrc(row0, p.v_end);
#pragma unroll
      for (int i = 0; i < N; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (LDS void*)(dst + i * 1024), 16,
                                                 off0 + (uint32_t)(ROWS * i) * (uint32_t)v_st_b, 0, 0, 0);
    }
  }

  // ---------------------------------------------------------------- DQ: K dequantized into BF16 LDS
  // Block b of K (FP8 payload and scale words) into registers: lane L of wave w stages 16-byte
  // chunk L % 8 of key rows 32w + 8i + L / 8 (i = 0..3) and those rows' scale words. Buffer loads
  // whose range ends at the tensor's last byte: rows past the end read zeros (and are masked).
  __device__ __forceinline__ void dq_load_k(int b) {
    const auto r = rsrc(kbase + (int64_t)(b * BN + 32 * wave) * k_st_b, p.k_end);
    const int r8 = lane >> 3;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = 8 * i + r8;
      kpre[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                              r, (int)((uint32_t)(row * (int)k_st_b) + 16u * (lane & 7)), 0, 0));
      // the scale storage is padded to whole 128-row blocks per sequence: every row exists
      kpre_sc[i] = *reinterpret_cast<const uint32_t*>(ksc_base + (int64_t)(b * BN + 32 * wave + row) * H * 4);
    }
  }

  // The staged chunks, dequantized exactly (E4M3 times the block's power of two) to BF16, into K
  // buffer buf in the BF16 layout that the scores read: row r holds 16 chunks of 8 elements, chunk c
  // at position c ^ (r % 16). A staged 16-byte FP8 chunk c8 becomes BF16 chunks 2 c8 and 2 c8 + 1.
  __device__ __forceinline__ void dq_store_k(int buf) {
    const int r8 = lane >> 3, c8 = lane & 7;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = 32 * wave + 8 * i + r8;
      const float sc = e8m0_to_float((kpre_sc[i] >> (8 * (c8 >> 1))) & 0xFFu);   // block c8 / 2 of the row
      const v8bf lo = fp8x8_to_bf16(kpre[i].x, kpre[i].y, sc), hi = fp8x8_to_bf16(kpre[i].z, kpre[i].w, sc);
      const uint32_t base = L::OFF_K + buf * L::K_BYTES + row * 256;
      *reinterpret_cast<LDS v8bf*>(dyn() + opaque(base + 16 * ((2 * c8) ^ (row & 15)))) = lo;
      *reinterpret_cast<LDS v8bf*>(dyn() + opaque(base + 16 * ((2 * c8 + 1) ^ (row & 15)))) = hi;
    }
  }

  // ---------------------------------------------------------------- precision guard
  // The whole tile may use the FP8 score path when c * max|q| * max|k| <= p.guard (16 unless the
  // caller sets another threshold) with
  // max|q| over the workgroup's queries and max|k| over all keys of the (sequence, head). In MX
  // mode both bounds come from the E8M0 scales (block maxima lie in (224, 448] * 2^e); in
  // per-tensor mode |q| is read from the codes and |k| from the cast's per-16-row code maxima
  // (the E4M3 range 448 without them).
  // Three parts: the first batch of K scale words is loaded before any other load of the tile
  // (its latency overlaps theirs); each wave publishes its bounds into the reduction slots before
  // the barrier that precedes the key loop; every wave combines them after that barrier.
  // The K data the guard reads: element i is the maximum scale byte of key rows 16i..16i+15 of
  // the sequence (MX, from the quantizer: ceil(Lk/16) elements), the largest E4M3 code magnitude
  // of packed rows 16(g0 + i)..16(g0 + i)+15 (per-tensor, from the cast: the groups that hold the
  // sequence's keys, neighbouring sequences' rows included), or the scale word of key row i (MX
  // without maxima: Lk elements).
  __device__ __forceinline__ int guard_count() const { return gcount; }
  __device__ __forceinline__ uint32_t guard_elem(int i) const {
    return kgm_base ? (uint32_t)kgm_base[(int64_t)i * H] : *reinterpret_cast<const uint32_t*>(ksc_base + (int64_t)i * H * 4);
  }
  // Branch-free, so that the eight loads go out together: an index past the end reads the last
  // element again, which leaves the maximum unchanged (and the values are not used before the
  // reduction, so nothing waits for them here).
  __device__ __forceinline__ void guard_prefetch() {
    const int n = guard_count();
#pragma unroll
    for (int u = 0; u < 8; ++u) ksw[u] = 0u;
    if (n == 0) return;
    if (kgm_base) {
#pragma unroll
      for (int u = 0; u < 8; ++u)
        ksw[u] = kgm_base[(int64_t)min((int)threadIdx.x + u * 256 * G, n - 1) * H];
    } else {
#pragma unroll
      for (int u = 0; u < 8; ++u)
        ksw[u] = *reinterpret_cast<const uint32_t*>(ksc_base + (int64_t)min((int)threadIdx.x + u * 256 * G, n - 1) * H * 4);
    }
  }

  // The sequence's offsets, loaded together (one memory round trip) and kept in scalar registers.
  __device__ __forceinline__ void load_meta() {
    const int q0 = p.cu_q[seq], q1 = p.cu_q[seq + 1], k0 = p.cu_k[seq], k1 = p.cu_k[seq + 1];
    const int sq = MX ? p.cu_scale_q[seq] : 0, sk = MX ? p.cu_scale_k[seq] : 0;
    q_start = __builtin_amdgcn_readfirstlane(q0);
    Lq = __builtin_amdgcn_readfirstlane(q1) - q_start;
    k_start = __builtin_amdgcn_readfirstlane(k0);
    Lk = __builtin_amdgcn_readfirstlane(k1) - k_start;
    scq = __builtin_amdgcn_readfirstlane(sq);
    sck = __builtin_amdgcn_readfirstlane(sk);
  }

  __device__ __forceinline__ void guard_publish(float* red) {
    float kbound = 448.0f;  // per-tensor mode without K maxima: the E4M3 range
    if (MX || kgm_base != nullptr) {  // uniform over the workgroup
      uint32_t m = 0;
#pragma unroll
      for (int u = 0; u < 8; ++u)
        m = max(m, max(max(ksw[u] & 0xFF, (ksw[u] >> 8) & 0xFF), max((ksw[u] >> 16) & 0xFF, ksw[u] >> 24)));
      // further batches (elements beyond the first 8 * 256 * G), 8 independent loads in flight each
      const int n = guard_count();
      for (int i0 = threadIdx.x + 8 * 256 * G; i0 < n; i0 += 8 * 256 * G) {
        uint32_t w[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int i = i0 + u * 256 * G;
          w[u] = i < n ? guard_elem(i) : 0u;
        }
#pragma unroll
        for (int u = 0; u < 8; ++u)
          m = max(m, max(max(w[u] & 0xFF, (w[u] >> 8) & 0xFF), max((w[u] >> 16) & 0xFF, w[u] >> 24)));
      }
      const uint32_t mm = wave_max_u32(m);
      // MX: block maxima lie in (224, 448] * 2^e; per-tensor: the largest code's value
      kbound = MX ? 448.0f * e8m0_to_float(mm) : __builtin_amdgcn_cvt_f32_fp8((int)mm, 0);
    }
    // per-wave bounds (each wave scanned a share of the key rows), combined after the
    // workgroup's next barrier by fp8_scores_ok_tile
    if (lane == 0) {
      red[threadIdx.x >> 6] = qbound;
      red[8 + (threadIdx.x >> 6)] = kbound;
    }
  }

  __device__ __forceinline__ bool fp8_scores_ok_tile(const float* red) const {
    float qb = 0.0f, kb = 0.0f;
#pragma unroll
    for (int w = 0; w < 4 * G; ++w) {
      qb = fmaxf(qb, red[w]);
      kb = fmaxf(kb, red[8 + w]);
    }
    return c * qb * kb <= p.guard;  // a negative threshold: never
  }

  // ---------------------------------------------------------------- scores
  // The score instructions' Q operands: held in registers by the two-group kernel (16 KB less
  // LDS read per key block and wave: 26.9 -> 26.3 us at the dense 2048 x 16 shape, 27.4 -> 26.5 us
  // with MX V), else read from LDS.
  __device__ __forceinline__ void q_frags(v8i qf[2]) const {
    if constexpr (QREG) {
      qf[0] = qreg[0];
      qf[1] = qreg[1];
    } else {
      qf[0] = q_frag(0);
      qf[1] = q_frag(1);
    }
  }

  // This wave's Q fragment for query tile nt (16 queries), from LDS.
  __device__ __forceinline__ v8i q_frag(int nt) const {
    LDS const v4u_t* qa;
    if constexpr (G == 1)
      qa = reinterpret_cast<LDS const v4u_t*>(dyn() + opaque(L::OFF_Q + (wave * 2 + nt) * 2048 + lane * 16));
    else
      qa = lds_at<const v4u_t>(lds_base - grp * L::GROUP_BYTES + L::OFF_Q + (wave * 2 + nt) * 2048 + lane * 16);
    return make_v8i(qa[0], qa[64]);   // + 1024 bytes
  }

  // BF16 scores of the block in K buffer buf from BF16 K and Q (QB): per key tile, 4 slices of 32
  // along head_dim; lane (n, g) reads key row 16t + n, slice u's chunk 4u + g (swizzled).
  __device__ __forceinline__ void scores_qb(int buf, v4f s[8][2]) {
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) {
      v4f acc[2] = {v4f{0.0f, 0.0f, 0.0f, 0.0f}, v4f{0.0f, 0.0f, 0.0f, 0.0f}};
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const v8bf kf = *lds_at<const v8bf>(lds_base + L::OFF_K + buf * L::K_BYTES + (16 * mt + n16) * 256 +
                                            16 * ((4 * u + g) ^ n16));
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qb16[nt][u], acc[nt], 0, 0, 0);
      }
      s[mt][0] = acc[0];
      s[mt][1] = acc[1];
      region_end();
    }
  }

  __device__ __forceinline__ void scores_fp8(int buf, v4f s[8][2]) {
    v8i qf[2];
    q_frags(qf);
    const uint32_t kt = lds_base + L::OFF_K + buf * L::K_BYTES;
    LDS const uint8_t* ksc = lds_at<const uint8_t>(lds_base + L::OFF_KSC + buf * L::KSC_BYTES + 4 * n16 + g);
    LDS const v4u_t* k_a = lds_at<const v4u_t>(kt + n16 * 128 + ((g ^ (n16 & 7)) << 4));
    LDS const v4u_t* k_b = lds_at<const v4u_t>(kt + n16 * 128 + (((4 + g) ^ (n16 & 7)) << 4));
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) {
      const v8i kf = make_v8i(k_a[mt * 128], k_b[mt * 128]);
      const int ks = MX ? (int)ksc[64 * mt] : 127;
#pragma unroll
      for (int nt = 0; nt < 2; ++nt)
        s[mt][nt] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(kf, qf[nt], v4f{0.0f, 0.0f, 0.0f, 0.0f},
                                                                     0, 0, 0, ks, 0, qsc[nt]);
    }
  }

  // Guarded path: scores from exactly dequantized BF16 operands, one 32-wide slice of head_dim
  // at a time (Q's slice reloaded from global memory, so only 8 registers hold it).
  __device__ __forceinline__ void scores_bf16(int buf, v4f s[8][2]) {
    const uint8_t* kt = lds + L::OFF_K + buf * L::K_BYTES;
    const uint32_t* ksc = reinterpret_cast<const uint32_t*>(lds + L::OFF_KSC + buf * L::KSC_BYTES);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      v8bf qb[2];  // B operand: lane (n, g) holds d = 32u + 8g + 0..7
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        uint2 w = make_uint2(0, 0);
        if (qrow[nt] != nullptr) w = ldg8(qrow[nt] + 32 * u + 8 * g);
        qb[nt] = fp8x8_to_bf16(w.x, w.y, e8m0_to_float((qsw[nt] >> (8 * u)) & 0xFFu));
      }
#pragma unroll
      for (int mt = 0; mt < 8; ++mt) {
        const int r = 16 * mt + n16;
        const uint32_t sw = MX ? ksc[r] : 0x7F7F7F7Fu;
        const int chunk = (2 * u + (g >> 1)) ^ (n16 & 7);
        const uint2 w = *reinterpret_cast<const uint2*>(kt + r * 128 + chunk * 16 + 8 * (g & 1));
        const v8bf kf = fp8x8_to_bf16(w.x, w.y, e8m0_to_float((sw >> (8 * u)) & 0xFFu));
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
          s[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qb[nt], u == 0 ? v4f{0.0f, 0.0f, 0.0f, 0.0f} : s[mt][nt], 0, 0, 0);
        region_end();
      }
    }
  }

  // ---------------------------------------------------------------- P V
  // O^T d tile dt += V^T P^T for the block in the V buffer at v_lane (this lane's LDS byte
  // address for d tile 0), V read transposed from the natural-layout tile.
  // fp8 V^T fragment of d tile dt (4 transposed reads)
  __device__ __forceinline__ v8i v_frag8(LDS uint8_t* v_lane, int dt, int jj) const {
    LDS v2i_t* base = reinterpret_cast<LDS v2i_t*>(v_lane + ((dt ^ jj) << 4));
    v8i vf;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const v2i_t w = __builtin_amdgcn_ds_read_tr8_b64_v2i32(base + r * 512);  // + r * 4096 bytes
      vf[2 * r] = w[0];
      vf[2 * r + 1] = w[1];
    }
    return vf;
  }

  __device__ __forceinline__ void pv_tile(LDS uint8_t* v_lane, int dt, int jj, const PF& pf) {
    if constexpr (FP8V) {
      LDS v2i_t* base = reinterpret_cast<LDS v2i_t*>(v_lane + ((dt ^ jj) << 4));
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
      LDS v4s_t* base = reinterpret_cast<LDS v4s_t*>(v_lane + ((dt ^ jj) << 5));
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const v2u_t w0 = __builtin_bit_cast(v2u_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16(base + (32 * u) * 32));  // (32u) rows * 256 B
        const v2u_t w1 = __builtin_bit_cast(v2u_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16(base + (32 * u + 16) * 32));
        const v8bf vf = __builtin_bit_cast(v8bf, make_uint4(w0[0], w0[1], w1[0], w1[1]));
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
          const uint4 w = make_uint4(pf.w[u][nt][0], pf.w[u][nt][1], pf.w[u][nt][2], pf.w[u][nt][3]);
          o[dt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, __builtin_bit_cast(v8bf, w), o[dt][nt], 0, 0, 0);
        }
      }
    }
  }

  // this lane's LDS address for d tile 0 of V buffer y in V object OBJ
  template <int OBJ>
  __device__ __forceinline__ LDS uint8_t* v_lane_addr(int y) const {
    const int jj = FP8V ? (n16 >> 1) : (n16 >> 2);
    const uint32_t off = y * L::V_BYTES + (FP8V ? (16 * (jj >> 2) + 4 * g + (jj & 3)) * 128 + 8 * (n16 & 1)
                                                : (4 * g + jj) * 256 + 8 * (n16 & 1) + 16 * ((n16 & 3) >> 1));
    if constexpr (G == 1) return vobj[OBJ] + opaque(off);
    return lds_at<uint8_t>((uint32_t)(uintptr_t)vobj[OBJ] + off);
  }

  // o_sum += 1^T P^T: the rounded probabilities summed on the matrix core with an all-ones
  // V^T tile, so O can be normalised by exactly the weights it was accumulated with.
  __device__ __forceinline__ void pv_sum(const PF& pf) {
    if constexpr (FP8V) {
      const v8i ones = {0x38383838, 0x38383838, 0x38383838, 0x38383838,
                        0x38383838, 0x38383838, 0x38383838, 0x38383838};  // E4M3 1.0
#pragma unroll
      for (int nt = 0; nt < 2; ++nt)
        o_sum[nt] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(ones, pf.f8[nt], o_sum[nt], 0, 0, 0, 127, 0, 127);
    } else {
      const v8bf ones = __builtin_bit_cast(v8bf, make_uint4(0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u));
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
          const uint4 w = make_uint4(pf.w[u][nt][0], pf.w[u][nt][1], pf.w[u][nt][2], pf.w[u][nt][3]);
          o_sum[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, __builtin_bit_cast(v8bf, w), o_sum[nt], 0, 0, 0);
        }
    }
  }

  // P V of a whole block resident in V buffer `buf`. One scheduling region per d tile, so that
  // the transposed V reads are not all hoisted ahead (that would hold 8 fragments at once).
  template <int OBJ>
  __device__ __forceinline__ void pv(int y, const PF& pf) {
    LDS uint8_t* v_lane = v_lane_addr<OBJ>(y);
    const int jj = FP8V ? (n16 >> 1) : (n16 >> 2);
    if constexpr (FP8V) {
      // software-pipelined: the transposed reads of d tile dt+1 are issued before the matrix
      // instructions of tile dt, so their latency overlaps. MX V: lane (n, g) supplies the
      // scale of V^T row 16 dt + n over the block's 32-key quarter g (the slot group g).
      LDS const uint8_t* vsc = lds_at<const uint8_t>(lds_base + L::OFF_VSC + y * L::VSC_BYTES + g * 128 + n16);
      v8i nxt = v_frag8(v_lane, 0, jj);
      int snxt = VMX ? (int)vsc[0] : 127;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        const v8i vf = nxt;
        const int sc = snxt;
        if (dt < 7) {
          nxt = v_frag8(v_lane, dt + 1, jj);
          if (VMX) snxt = (int)vsc[16 * (dt + 1)];
        }
        region_end();
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
          o[dt][nt] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(vf, pf.f8[nt], o[dt][nt], 0, 0, 0, sc, 0, 127);
      }
    } else {
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        pv_tile(v_lane, dt, jj, pf);
        region_end();
      }
    }
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

  // ---------------------------------------------------------------- two-group phases
  // Probabilities of key block (scores in s) against the running maximum m_run: pf <- the packed
  // probabilities, rs <- this lane's unrounded sums over its keys of each row.
  __device__ __forceinline__ void probs(const v4f s[8][2], PF& pf, float rs[2]) const {
    rs[0] = rs[1] = 0.0f;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        float pk[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          pk[i] = __builtin_amdgcn_exp2f(fmaf(s[k][nt][i], c, -m_run[nt]));
          rs[nt] += pk[i];
        }
        if constexpr (FP8V) {
          pf.f8[nt][k] = (int)cvt4_e4m3_over((uint32_t)pf.f8[nt][k], pk[0], pk[1], pk[2], pk[3]);
        } else {
          pf.w[k >> 1][nt][2 * (k & 1)] = cvt_pk_bf16(pk[0], pk[1]);
          pf.w[k >> 1][nt][2 * (k & 1) + 1] = cvt_pk_bf16(pk[2], pk[3]);
        }
      }
    }
  }

  // Softmax of key block b (scores in s): mask, lazy running maximum, probabilities -> pf,
  // unrounded row sums -> l_run. The maximum is only taken when needed: the probabilities are
  // first formed against the current m_run, and each lane's sum over its keys of a row bounds
  // every probability it holds, so when no such sum exceeds 2^8 none of them does and the block
  // is done. Otherwise (and on the wave's first block, when m_run is still -inf) the block's row
  // maxima move m_run, O and the rounded sum are rescaled at once (O holds exactly the P V of the
  // earlier blocks here), and the probabilities are formed again.
  template <bool FIRST>
  __device__ __forceinline__ void softmax(int b, bool mask, v4f s[8][2], PF& pf) {
    if (mask) {  // wave-uniform: the block runs past the last key
      const int kb = b * BN;
#pragma unroll
      for (int mt = 0; mt < 8; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (kb + 64 * (mt >> 2) + 16 * g + 4 * (mt & 3) + i >= Lk) {  // the key order of dma_k
            s[mt][0][i] = -INFINITY;
            s[mt][1][i] = -INFINITY;
          }
    }
    float rs[2];
    bool exact = FIRST;
    if (!FIRST) {
      probs(s, pf, rs);
      exact = __ballot(!(rs[0] <= LAZY_SUM) || !(rs[1] <= LAZY_SUM)) != 0;  // wave-uniform
    }
    if (exact) {
      float alpha[2];
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        float mx = fmaxf(s[0][nt][0], s[0][nt][1]);
#pragma unroll
        for (int mt = 0; mt < 8; ++mt)
#pragma unroll
          for (int i = (mt == 0 ? 2 : 0); i < 4; i += 2) mx = fmaxf(mx, fmaxf(s[mt][nt][i], s[mt][nt][i + 1]));
        const float m_new = fmaxf(m_run[nt], xmax16_32(mx) * c);
        alpha[nt] = __builtin_amdgcn_exp2f(m_run[nt] - m_new);
        l_run[nt] *= alpha[nt];
        m_run[nt] = m_new;
      }
      if (!FIRST) rescale(alpha);
      probs(s, pf, rs);
    }
    l_run[0] += rs[0];
    l_run[1] += rs[1];
  }

  // FP8 scores of the block in K buffer kbuf into s, one key tile per scheduling region.
  __device__ __forceinline__ void qk(int kbuf, v4f s[8][2]) {
    v8i qf[2];
    q_frags(qf);
    const uint32_t kt = lds_base + L::OFF_K + kbuf * L::K_BYTES;
    LDS const uint8_t* ksc = lds_at<const uint8_t>(lds_base + L::OFF_KSC + kbuf * L::KSC_BYTES + 4 * n16 + g);
    LDS const v4u_t* k_a = lds_at<const v4u_t>(kt + n16 * 128 + ((g ^ (n16 & 7)) << 4));
    LDS const v4u_t* k_b = lds_at<const v4u_t>(kt + n16 * 128 + (((4 + g) ^ (n16 & 7)) << 4));
    // software-pipelined like pv(): key tile t+1's reads go out before tile t's instructions
    v8i kn = make_v8i(k_a[0], k_b[0]);
    int ksn = MX ? (int)ksc[0] : 127;
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const v8i kf = kn;
      const int ks = ksn;
      if (t < 7) {
        kn = make_v8i(k_a[(t + 1) * 128], k_b[(t + 1) * 128]);      // + 2048 bytes per tile
        ksn = MX ? (int)ksc[64 * (t + 1)] : 127;
      }
      region_end();
#pragma unroll
      for (int nt = 0; nt < 2; ++nt)
        s[t][nt] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(kf, qf[nt], v4f{0.0f, 0.0f, 0.0f, 0.0f},
                                                                    0, 0, 0, ks, 0, qsc[nt]);
    }
  }

  // ---------------------------------------------------------------- one pipeline step
  // Softmax of local block j (scores in s -> probabilities in pf_cur), scores of block j+1
  // written back into s (if DO_QK) and O += P(j-1) V(j-1) (if DO_PV). Issued as 8 slots: slot k
  // turns score tile k into probabilities, then overwrites it with the next block's score tile
  // k, and runs the P V instructions of d tile k, so matrix and vector work overlap and live
  // ranges stay short.
  template <bool DO_QK, bool DO_PV, bool MASK, int PAR>
  __device__ __forceinline__ void step(int j, v4f s[8][2], const PF& pf_prev, PF& pf_cur) {
    if (MASK) {
      const int kb = blk(j) * BN;
#pragma unroll
      for (int mt = 0; mt < 8; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (kb + 16 * mt + 4 * g + i >= Lk) {
            s[mt][0][i] = -INFINITY;
            s[mt][1][i] = -INFINITY;
          }
    }
    // Row maxima of the block. The running maximum m_run only moves when some row of the wave
    // exceeds it by more than LAZY_LOG2; otherwise the probabilities are taken against the stale
    // maximum and O needs no rescale.
    float cand[2];
    bool move = false;
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      float mx = fmaxf(s[0][nt][0], s[0][nt][1]);
#pragma unroll
      for (int mt = 0; mt < 8; ++mt)
#pragma unroll
        for (int i = (mt == 0 ? 2 : 0); i < 4; i += 2) mx = fmaxf(mx, fmaxf(s[mt][nt][i], s[mt][nt][i + 1]));
      mx = xmax16_32(mx);
      cand[nt] = mx * c;
      move = move || (cand[nt] > m_run[nt] + LAZY_LOG2);
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

    const int kb1 = (j + 1) & 1;
    LDS const uint8_t* ksc = dyn() + opaque(L::OFF_KSC + kb1 * L::KSC_BYTES + 4 * n16 + g);
    LDS const v4u_t* k_a = reinterpret_cast<LDS const v4u_t*>(
        dyn() + opaque(L::OFF_K + kb1 * L::K_BYTES + n16 * 128 + ((g ^ (n16 & 7)) << 4)));
    LDS const v4u_t* k_b = reinterpret_cast<LDS const v4u_t*>(
        dyn() + opaque(L::OFF_K + kb1 * L::K_BYTES + n16 * 128 + (((4 + g) ^ (n16 & 7)) << 4)));
    LDS uint8_t* v_lane = v_lane_addr<1 - PAR>(0);   // V of the previous block
    const int jj = FP8V ? (n16 >> 1) : (n16 >> 2);
    v8i qf[2];
    v8i kn;   // FP8 scores: the next key tile's fragment and scale, read one slot ahead (their
    int ksn;  // latency passes under a slot's vector work)
    if (DO_QK && !KB16) {
      qf[0] = q_frag(0);
      qf[1] = q_frag(1);
      kn = make_v8i(k_a[0], k_b[0]);
      ksn = MX ? (int)ksc[0] : 127;
    }
    LDS const v8bf* kq[4];  // QB, DQ: this lane's slice-u chunk of key row n16 (row 16t + n16: + t * 4096 bytes)
    if constexpr (KB16) {
#pragma unroll
      for (int u = 0; u < 4; ++u)
        kq[u] = reinterpret_cast<LDS const v8bf*>(dyn() + opaque(L::OFF_K + kb1 * L::K_BYTES + n16 * 256 +
                                                                 16 * ((4 * u + g) ^ n16)));
    }

    float rs[2] = {0.0f, 0.0f};
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      // FP8 scores: this slot's key tile fragment was read one slot ahead; key tile k+1's reads go
      // out now, ahead of this slot's vector work
      v8i kf;
      int ks = 127;
      if (DO_QK && !KB16) {
        kf = kn;
        ks = ksn;
        if (k < 7) {
          kn = make_v8i(k_a[(k + 1) * 128], k_b[(k + 1) * 128]);  // + 2048 bytes per tile
          ksn = MX ? (int)ksc[64 * (k + 1)] : 127;
        }
      }
      // probabilities of score tile k of block j
#pragma unroll
      for (int nt = 0; nt < 2; ++nt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float pv = __builtin_amdgcn_exp2f(fmaf(s[k][nt][i], c, -m_use[nt]));
          s[k][nt][i] = pv;
          rs[nt] += pv;
        }
      if constexpr (FP8V) {
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
          pf_cur.f8[nt][k] = (int)cvt4_e4m3(s[k][nt][0], s[k][nt][1], s[k][nt][2], s[k][nt][3]);
      } else {
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
          pf_cur.w[k >> 1][nt][2 * (k & 1)] = cvt_pk_bf16(s[k][nt][0], s[k][nt][1]);
          pf_cur.w[k >> 1][nt][2 * (k & 1) + 1] = cvt_pk_bf16(s[k][nt][2], s[k][nt][3]);
        }
      }
      if (DO_QK && KB16) {  // BF16 scores of block j+1, key tile k
        v4f acc[2] = {v4f{0.0f, 0.0f, 0.0f, 0.0f}, v4f{0.0f, 0.0f, 0.0f, 0.0f}};
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const v8bf kf = kq[u][k * 256];  // + k * 4096 bytes
#pragma unroll
          for (int nt = 0; nt < 2; ++nt) acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qb16[nt][u], acc[nt], 0, 0, 0);
        }
        s[k][0] = acc[0];
        s[k][1] = acc[1];
      } else if (DO_QK) {  // scores of block j+1, key tile k (overwrites the consumed tile)
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

  // ---------------------------------------------------------------- key loop
  // One group (BF16 V). Local iteration j = key block j: loads K of block j+2 into K buffer j%2
  // (freed when the scores of block j were taken) and V of block j into V buffer j%2 (freed by
  // the P V of block j-2 in the previous iteration), runs the pipelined step (scores of block j+1
  // on the FP8 path when FAST, else by the BF16 path after the step; P V of block j-1 inside the
  // step's slots), then waits for its loads and synchronises the workgroup.
  // PAR = j % 2 (a constant: the V buffers are chosen at compile time).
  template <bool FAST, bool FIRST, bool LAST, int PAR>
  __device__ __forceinline__ void iteration1(int j, v4f s[8][2], const PF& pf_prev, PF& pf_cur) {
    if constexpr (DQ && !DQS) {
      if (j + 2 < ng) dq_load_k(blk(j + 2));
    } else {
      if (j + 2 < ng) dma_k(0, blk(j + 2), j & 1);
    }
    dma_v(PAR, blk(j), 0);
    step<FAST && !LAST, !FIRST, LAST, PAR>(j, s, pf_prev, pf_cur);
    if (!FAST && !LAST) scores_bf16((j + 1) & 1, s);
    if constexpr (DQ && !DQS) {  // block j+2's K, staged in registers during the step, into K buffer j % 2
      if (j + 2 < ng) dq_store_k(j & 1);
    }
    wait_vm_all();
    __syncthreads();
  }

  // Two groups (E4M3 V), local iteration j = key block blk(j) of this group. Both groups do
  // one softmax (VALU phase) and the P V and score instructions (matrix phase) per iteration,
  // in opposite order, so that on each SIMD one wave's softmax meets the other wave's matrix
  // instructions:
  //   group 0: softmax(j), P V(j), scores(j+1)
  //   group 1: P V(j-1), scores(j), then the loads of both groups, then softmax(j)
  // A wave's LDS reads must wait for every load into LDS that the wave itself has in flight, so
  // group 1 issues all loads after its last LDS read of the iteration (they land during its
  // softmax) and group 0 issues none (issuing group 0's own loads from group 0 instead slows its
  // score phase). Targets: group 0's K(j+2) -> its K buffer j%2 and V(j+1) -> its V buffer
  // (j+1)%2; group 1's K(j+1) -> (j+1)%2 and V(j) -> j%2: each was last read in the previous
  // iteration. Every iteration ends with its loads complete and one barrier.
  template <int GRP, bool FAST, bool FIRST>
  __device__ __forceinline__ void iteration2(int j, v4f s[8][2], PF& pf) {
    const bool last = j == ng - 1;
    const bool mask = last && (Lk & (BN - 1)) != 0;
    if constexpr (GRP == 0) {
      softmax<FIRST>(blk(j), mask, s, pf);
      pv<0>(j & 1, pf);
      if (!last) {
        if (FAST) qk((j + 1) & 1, s); else scores_bf16((j + 1) & 1, s);
      }
      if (j + 2 < ng) dma_k(0, blk(j + 2), j & 1);
      if (j + 1 < ng) dma_v(0, blk(j + 1), (j + 1) & 1);
    } else {
      if (!FIRST) pv<1>((j + 1) & 1, pf);
      if (FAST) qk(j & 1, s); else scores_bf16(j & 1, s);
      if (j + 1 < ng) dma_k(1, blk(j + 1), (j + 1) & 1);
      dma_v(1, blk(j), j & 1);
      softmax<FIRST>(blk(j), mask, s, pf);
    }
    wait_vm_all();
    __syncthreads();
  }

  // niter: iterations of the group with the most blocks; a group with fewer blocks only takes
  // part in the barriers of the remaining iterations.
  template <bool FAST>
  __device__ __forceinline__ void main_loop(int niter) {
    v4f s[8][2];
    int j = 0;
    if constexpr (G == 1) {
      if (ng > 0) {
        if constexpr (KB16)
          scores_qb(0, s);
        else if (FAST)
          scores_fp8(0, s);
        else
          scores_bf16(0, s);
      }
      __syncthreads();  // K buffer 0 is reused for blk(2)
      // iteration j writes its probabilities to pa (j even) or pb (j odd) and reads the
      // previous block's from the other set
      PF pa, pb;
      if (ng == 1) {
        iteration1<FAST, true, true, 0>(0, s, pb, pa);
      } else {
        iteration1<FAST, true, false, 0>(0, s, pb, pa);
        for (j = 1; j + 1 < ng - 1; j += 2) {
          iteration1<FAST, false, false, 1>(j, s, pa, pb);
          iteration1<FAST, false, false, 0>(j + 1, s, pb, pa);
        }
        if (j == ng - 2) {
          iteration1<FAST, false, false, 1>(j, s, pa, pb);
          iteration1<FAST, false, true, 0>(j + 1, s, pb, pa);
        } else {
          iteration1<FAST, false, true, 1>(j, s, pa, pb);
        }
      }
      // the last block's P V (V buffer (ng-1)%2; probabilities in pa when ng is odd, else pb)
      if (ng & 1) pv<0>(0, pa);
      else pv<1>(0, pb);
    } else {
      // separate loops per group (the order of work differs), each register-allocated alone.
      // Group 0 takes the scores of its first block here (group 1 inside its first iteration),
      // inside its own branch so that no score tile is live across the split; one barrier each
      // (K buffer 0 is reused for blk(2)).
      if (grp == 0) {
        if (ng > 0) {
          if (FAST) scores_fp8(0, s); else scores_bf16(0, s);
        }
        __syncthreads();
        loop2<0, FAST>(s, niter);
      } else {
        __syncthreads();
        loop2<1, FAST>(s, niter);
      }
    }
  }

  template <int GRP, bool FAST>
  __device__ __forceinline__ void loop2(v4f s[8][2], int niter) {
    PF pf{};  // defined contents: the packing writes over the previous probabilities
    int j = 0;
    if (ng > 0) {
      iteration2<GRP, FAST, true>(0, s, pf);
      for (j = 1; j < ng; ++j) iteration2<GRP, FAST, false>(j, s, pf);
    }
    // group 1 still owes the P V of its last block: in the spare iteration if there is one
    bool owed = GRP == 1 && ng > 0;
    for (; j < niter; ++j) {
      if (owed) {
        pv<GRP>((ng - 1) & 1, pf);
        owed = false;
      }
      __syncthreads();
    }
    if (owed) pv<GRP>((ng - 1) & 1, pf);
  }

  // ---------------------------------------------------------------- end of the tile
  // d tiles DT0..DT0+3 of O (both query halves) into the LDS area at `give` (lane-contiguous
  // 16-byte slots, 8 per lane).
  template <int DT0>
  __device__ __forceinline__ void give_half(LDS v4f* give) const {
#pragma unroll
    for (int d = 0; d < 4; ++d)
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) give[(2 * d + nt) * 64] = o[DT0 + d][nt];
  }

  // Combines this group's state with the other group's (m, l, rounded sum) in ml/os and its
  // half of O at `take` (d tiles 0-3 for group 0, 4-7 for group 1). Every sum takes group 0's
  // term first, so both groups compute the same l, rounded sum and m.
  template <int GRP>
  __device__ __forceinline__ void merge_half(const LDS v4f* take, const v4f ml, const v4f os) {
    float aw[2], at[2];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      const float m = fmaxf(m_run[nt], ml[nt]);      // finite: group 0 has at least one block
      aw[nt] = __builtin_amdgcn_exp2f(m_run[nt] - m);
      at[nt] = __builtin_amdgcn_exp2f(ml[nt] - m);   // 0 for a group with no block (-inf)
      const float w0 = GRP == 0 ? aw[nt] : at[nt], w1 = GRP == 0 ? at[nt] : aw[nt];
      const float l0 = GRP == 0 ? l_run[nt] : ml[2 + nt], l1 = GRP == 0 ? ml[2 + nt] : l_run[nt];
      const float s0 = GRP == 0 ? o_sum[nt][0] : os[nt], s1 = GRP == 0 ? os[nt] : o_sum[nt][0];
      l_run[nt] = l0 * w0 + l1 * w1;
      o_sum[nt][0] = s0 * w0 + s1 * w1;
      m_run[nt] = m;
    }
    constexpr int DT0 = GRP == 0 ? 0 : 4;
#pragma unroll
    for (int d = 0; d < 4; ++d)
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        const v4f t = take[(2 * d + nt) * 64];
        o[DT0 + d][nt] = GRP == 0 ? o[DT0 + d][nt] * aw[nt] + t * at[nt] : t * at[nt] + o[DT0 + d][nt] * aw[nt];
      }
  }

  // O = O^T / (rounded sum) * vd -> BF16 and LSE = ln2 * (m + log2 l), as in epilogue() below.
  // Two-group kernel: this group's half of O (d tiles DT0..DT0+3 = 64 columns) for the wave's 32
  // queries, staged through the group's V object (free once the key loop is over: every wave
  // has passed the merge barrier) so that each store writes 8 whole 128-byte row halves instead
  // of 16 32-byte pieces. Row r of the stage holds query wave*32 + r; its 16-byte chunk c sits at
  // chunk c ^ (r & 7).
  template <int DT0>
  __device__ __forceinline__ void epilogue_staged(float vd, bool with_lse) {
    const int q0 = qtile0 * BM;
    LDS uint8_t* stg = vobj[DT0 == 0 ? 0 : 1] + wave * 4096;
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      float lt = l_run[nt] + __shfl_xor(l_run[nt], 16);
      lt += __shfl_xor(lt, 32);
      const int r = nt * 16 + n16;
      const int qi = q0 + wave * 32 + r;
      const float ls = o_sum[nt][0];
      const float inv = ls > 0.0f ? 1.0f / ls : 0.0f;
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const v4f x = o[DT0 + d][nt];
        const uint32_t u = (uint32_t)(4 * d + g) ^ (uint32_t)(2 * (r & 7));  // 8-byte unit in the row
        *reinterpret_cast<LDS v2u_t*>(stg + r * 128 + u * 8) =
            v2u_t{cvt_pk_bf16((x[0] * inv) * vd, (x[1] * inv) * vd), cvt_pk_bf16((x[2] * inv) * vd, (x[3] * inv) * vd)};
      }
      if (with_lse && g == 0 && qi < Lq)
        p.lse[(int64_t)head * p.total_q + q_start + qi] =
            lt > 0.0f ? (m_run[nt] + __builtin_amdgcn_logf(lt)) * LN2 : -INFINITY;
    }
    const int c = lane & 7;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int r = 8 * k + (lane >> 3);
      const v4u_t w = *reinterpret_cast<LDS const v4u_t*>(stg + r * 128 + ((c ^ (r & 7)) << 4));
      const int qi = q0 + wave * 32 + r;
      if (qi < Lq)
        *reinterpret_cast<uint4*>(p.out + ((int64_t)(q_start + qi) * H + head) * 128 + 16 * DT0 + 8 * c) =
            make_uint4(w[0], w[1], w[2], w[3]);
    }
  }

  // One-group kernel: the same staging for whole rows. Each wave writes its 32 queries' BF16 rows
  // (256 bytes) into 8 KB of V object 0 (the caller's barrier has ended every wave's V reads;
  // 16-byte chunk c of row r at c ^ (r & 15)) and stores them as 4 whole rows per instruction.
  __device__ __forceinline__ void epilogue_staged_rows(float vd) {
    const int q0 = qtile0 * BM;
    LDS uint8_t* stg = vobj[0] + wave * 8192;
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      float lt = l_run[nt] + __shfl_xor(l_run[nt], 16);
      lt += __shfl_xor(lt, 32);
      const int r = nt * 16 + n16;
      const int qi = q0 + wave * 32 + r;
      const float ls = o_sum[nt][0];
      const float inv = ls > 0.0f ? 1.0f / ls : 0.0f;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        const v4f x = o[dt][nt];
        const uint32_t u = (uint32_t)(4 * dt + g) ^ (uint32_t)(2 * (r & 15));  // 8-byte unit in the row
        *reinterpret_cast<LDS v2u_t*>(stg + r * 256 + u * 8) =
            v2u_t{cvt_pk_bf16((x[0] * inv) * vd, (x[1] * inv) * vd), cvt_pk_bf16((x[2] * inv) * vd, (x[3] * inv) * vd)};
      }
      if (g == 0 && qi < Lq)
        p.lse[(int64_t)head * p.total_q + q_start + qi] =
            lt > 0.0f ? (m_run[nt] + __builtin_amdgcn_logf(lt)) * LN2 : -INFINITY;
    }
    const int c = lane & 15;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int r = 4 * k + (lane >> 4);
      const v4u_t w = *reinterpret_cast<LDS const v4u_t*>(stg + r * 256 + ((c ^ (r & 15)) << 4));
      const int qi = q0 + wave * 32 + r;
      if (qi < Lq)
        *reinterpret_cast<uint4*>(p.out + ((int64_t)(q_start + qi) * H + head) * 128 + 8 * c) =
            make_uint4(w[0], w[1], w[2], w[3]);
    }
  }

  // O d tiles DT0..DT1-1 = O^T / (rounded sum) * vd -> BF16; with LSE, also
  // LSE = ln2 * (m + log2 l). (The two-group kernel's path for a tile with no key block.)
  template <int DT0, int DT1>
  __device__ __forceinline__ void epilogue(float vd, bool with_lse) {
    const int q0 = qtile0 * BM;
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      float lt = l_run[nt] + __shfl_xor(l_run[nt], 16);
      lt += __shfl_xor(lt, 32);
      const int qi = q0 + wave * 32 + nt * 16 + n16;
      if (qi < Lq) {
        const float ls = o_sum[nt][0];  // every row of the ones tile holds the rounded sum
        const float inv = ls > 0.0f ? 1.0f / ls : 0.0f;
        uint16_t* op = p.out + ((int64_t)(q_start + qi) * H + head) * 128 + 4 * g;
#pragma unroll
        for (int dt = DT0; dt < DT1; ++dt) {
          const v4f x = o[dt][nt];
          const uint2 w = make_uint2(cvt_pk_bf16((x[0] * inv) * vd, (x[1] * inv) * vd),
                                     cvt_pk_bf16((x[2] * inv) * vd, (x[3] * inv) * vd));
          *reinterpret_cast<uint2*>(op + 16 * dt) = w;
        }
        if (with_lse && g == 0)
          p.lse[(int64_t)head * p.total_q + q_start + qi] =
              lt > 0.0f ? (m_run[nt] + __builtin_amdgcn_logf(lt)) * LN2 : -INFINITY;
      }
    }
  }

  // One query tile. The precision guard decides before the key loop between FP8 and BF16
  // scores. MODE 2: both loops in this function. MODE 0: FP8 scores only; when the guard fails,
  // every wave returns false with no load in flight and nothing written, and the caller runs the
  // tile again with MODE 1 (BF16 scores, no guard: the two-group kernel's BF16 score loop, or
  // the DQ pipeline for the BF16-V kernel), which always completes and returns true.
  template <int MODE>
  __device__ __forceinline__ bool run(int qtile) {
    // MODE 3 (DQS only): the DQ pipeline started on speculation; it evaluates the guard in its
    // prologue, from loads it makes anyway, and returns false (no load in flight) if the tile may
    // take FP8 scores after all.
    static_assert(MODE != 3 || DQS, "speculative start: the DQ pipeline with K's BF16 values");
    constexpr bool GUARD = (MODE != 1 && !KB16) || MODE == 3;  // this call evaluates the guard
    constexpr bool MAY_SLOW = MODE != 0;  // this call may run the BF16 score loop
    // The one-group MX kernel decides before its first K and Q loads, from the Q scale words and
    // the K bound alone: a tile that fails then leaves at once for the DQ pipeline instead of
    // first loading and waiting for the FP8 path's operands.
    constexpr bool EARLY = MODE == 0 && G == 1 && MX && !KB16;
    H = p.num_heads;
    qtile0 = qtile;
    const int q0 = qtile * BM;
    nb = (Lk + BN - 1) / BN;
    ng = (nb - grp + G - 1) / G;
    const int niter = (nb + G - 1) / G;
    const int tid = threadIdx.x & 255;
    lane = tid & 63;
    // wave-uniform by construction; readfirstlane lets the compiler keep it (and everything
    // derived from it: buffer offsets, branches, loop bounds) in scalar registers
    wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    n16 = lane & 15;
    g = lane >> 4;

    const float qd = p.q_descale ? p.q_descale[seq * p.qd_ss + head * p.qd_sh] : 1.0f;
    const float kd = p.k_descale ? p.k_descale[seq * p.kd_ss + head * p.kd_sh] : 1.0f;
    c = (p.scale_log2 * qd) * kd;  // identical arithmetic with or without descales

    if constexpr (DQS) {  // K's quantized values as BF16: (total_k, H, 128) contiguous
      kbase = p.k_deq + ((int64_t)k_start * H + head) * 256;
      k_st_b = (int64_t)H * 256;
      kend = p.k_deq_end;
    } else {
      kbase = p.k + ((int64_t)k_start * p.k_st + (int64_t)head * p.k_sh) * (QB ? 2 : 1);
      k_st_b = p.k_st * (QB ? 2 : 1);
      kend = p.k_end;
    }
    vbase = reinterpret_cast<const uint8_t*>(p.v) + ((int64_t)k_start * p.v_st + (int64_t)head * p.v_sh) * (FP8V ? 1 : 2);
    v_st_b = p.v_st * (FP8V ? 1 : 2);
    ksc_base = MX ? p.k_scale + ((int64_t)sck * H + head) * 4 : nullptr;
    kgm_base = nullptr;
    gcount = Lk;
    if (p.k_gmax != nullptr && MX) {
      kgm_base = p.k_gmax + (int64_t)(sck / 16) * H + head;
      gcount = (Lk + 15) / 16;
    } else if (p.k_gmax != nullptr && Lk > 0) {
      const int g0 = k_start / 16;
      kgm_base = p.k_gmax + (int64_t)g0 * H + head;
      gcount = (k_start + Lk - 1) / 16 - g0 + 1;
    }
    if (GUARD && (MX || kgm_base != nullptr)) guard_prefetch();
    if constexpr (EARLY) {
      if (nb > 0) {
        uint32_t qms = 0;  // largest scale byte of the tile's queries (byte g of each row's word)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
          const int qi = q0 + wave * 32 + nt * 16 + n16;
          const bool in = qi < Lq;
          const uint32_t sw = *reinterpret_cast<const uint32_t*>(p.q_scale + (((int64_t)scq + (in ? qi : Lq - 1)) * H + head) * 4);
          qms = max(qms, in ? (sw >> (8 * g)) & 0xFFu : 0u);
        }
        qbound = 448.0f * e8m0_to_float(wave_max_u32(qms));
        float* red = reinterpret_cast<float*>(lds + L::OFF_RED);
        guard_publish(red);
        wait_vm_all();
        __syncthreads();
        if (!fp8_scores_ok_tile(red)) return false;  // uniform; no load in flight
      }
    }

    // start the first loads before touching Q
    if constexpr (DQS) {
      if (ng > 0) dma_k(0, blk(0), 0);
      if (ng > 1) dma_k(0, blk(1), 1);
    } else if constexpr (DQ) {
      if (ng > 0) dq_load_k(blk(0));  // stored as BF16 once Q's loads have gone out
    } else if (ng > 0) {
      if (grp == 0) {
        dma_k(0, blk(0), 0);
        if (ng > 1) dma_k(0, blk(1), 1);
        if (G == 2) dma_v(0, blk(0), 0);
      } else {
        dma_k(1, blk(0), 0);
      }
    }

    // ---- Q fragments: BF16 in registers (QB; DQ: dequantized exactly), or FP8 (score B operand)
    // in registers (QREG) or through LDS; the guarded path of the two-group kernel reloads FP8 Q
    // as BF16 ----
    if constexpr (DQ) {
      uint32_t qms = 0;  // MODE 3: largest scale byte of the tile's queries
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        const int qi = q0 + wave * 32 + nt * 16 + n16;
        const bool in = qi < Lq;
        const int qc = in ? qi : Lq - 1;
        const uint8_t* qp = p.q + (int64_t)(q_start + qc) * p.q_st + (int64_t)head * p.q_sh;
        const uint32_t sw = *reinterpret_cast<const uint32_t*>(p.q_scale + (((int64_t)scq + qc) * H + head) * 4);
        if (MODE == 3) qms = max(qms, in ? (sw >> (8 * g)) & 0xFFu : 0u);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          uint2 w = ldg8(qp + 32 * u + 8 * g);  // head_dim 32u + 8g .. 32u + 8g + 7: scale block u
          if (!in) w = make_uint2(0, 0);
          qb16[nt][u] = fp8x8_to_bf16(w.x, w.y, e8m0_to_float((sw >> (8 * u)) & 0xFFu));
        }
      }
      if (MODE == 3) qbound = 448.0f * e8m0_to_float(wave_max_u32(qms));
      if (!DQS && ng > 0) {
        dq_store_k(0);
        if (ng > 1) {
          dq_load_k(blk(1));
          dq_store_k(1);
        }
      }
    }
    if constexpr (QB) {
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        const int qi = q0 + wave * 32 + nt * 16 + n16;
        const bool in = qi < Lq;
        const uint16_t* qp = reinterpret_cast<const uint16_t*>(p.q) + (int64_t)(q_start + (in ? qi : Lq - 1)) * p.q_st +
                             (int64_t)head * p.q_sh;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          uint4 w = ldg16(qp + 32 * u + 8 * g);  // head_dim 32u + 8g .. 32u + 8g + 7
          if (!in) w = make_uint4(0, 0, 0, 0);
          qb16[nt][u] = __builtin_bit_cast(v8bf, w);
        }
      }
    }
    // Branch-free: a row past the sequence's end reads its last row (the tile has at least one)
    // and is then zeroed, so that every load goes out at once.
    uint32_t qmax_code = 0, qmax_scale = 0;
    v8i qf[2];
#pragma unroll
    for (int nt = 0; nt < 2 && !KB16; ++nt) {
      const int qi = q0 + wave * 32 + nt * 16 + n16;
      const bool in = qi < Lq;
      const int qc = in ? qi : Lq - 1;
      const uint8_t* qp = p.q + (int64_t)(q_start + qc) * p.q_st + (int64_t)head * p.q_sh;
      uint4 a = ldg16(qp + 16 * g), b = ldg16(qp + 64 + 16 * g);
      uint32_t sw = MX ? *reinterpret_cast<const uint32_t*>(p.q_scale + (((int64_t)scq + qc) * H + head) * 4) : 0x7F7F7F7Fu;
      if (!in) {
        a = make_uint4(0, 0, 0, 0);
        b = make_uint4(0, 0, 0, 0);
        sw = 0x7F7F7F7Fu;
      }
      qf[nt] = make_v8i(a, b);
      if (QREG) qreg[nt] = qf[nt];
      qsc[nt] = (int)((sw >> (8 * g)) & 0xFFu);
      if (MAY_SLOW) {
        qrow[nt] = in ? qp : nullptr;
        qsw[nt] = sw;
      }
      uint32_t words[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const uint32_t w = words[i] & 0x7F7F7F7Fu;
        qmax_code = max(qmax_code, max(max(w & 0xFF, (w >> 8) & 0xFF), max((w >> 16) & 0xFF, w >> 24)));
      }
      qmax_scale = max(qmax_scale, in ? (uint32_t)qsc[nt] : 0u);
    }
    if (grp == 0 && !KB16 && !QREG) {  // both groups hold the same queries: group 0 stores the fragments
      LDS v4u_t* qa = lds_at<v4u_t>(lds_base + L::OFF_Q + wave * 2 * 2048 + lane * 16);
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        qa[nt * 128] = v4u_t{(unsigned)qf[nt][0], (unsigned)qf[nt][1], (unsigned)qf[nt][2], (unsigned)qf[nt][3]};
        qa[nt * 128 + 64] = v4u_t{(unsigned)qf[nt][4], (unsigned)qf[nt][5], (unsigned)qf[nt][6], (unsigned)qf[nt][7]};
      }
    }
    if (!GUARD || EARLY || KB16) {
    } else if (MX) {
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
      float* red = reinterpret_cast<float*>(lds - grp * L::GROUP_BYTES + L::OFF_RED);
      if (GUARD && !EARLY) guard_publish(red);
      wait_vm_all();
      __syncthreads();
      if constexpr (KB16) {
        if constexpr (MODE == 3) {
          if (fp8_scores_ok_tile(red)) return false;  // uniform; every load has landed
        }
        main_loop<true>(niter);
      } else if constexpr (MODE == 1) {
        main_loop<false>(niter);
      } else if constexpr (MODE == 0) {
        if (!EARLY && !fp8_scores_ok_tile(red)) return false;  // uniform: every wave reads the same slots
        main_loop<true>(niter);
      } else {
        if (fp8_scores_ok_tile(red)) main_loop<true>(niter); else main_loop<false>(niter);
      }
    }

    const float vd = p.v_descale ? p.v_descale[seq * p.vd_ss + head * p.vd_sh] : 1.0f;
    if (G == 2 && nb > 0) {
      // Merge of the two groups' partial results, split by d tile: group 0 finishes d tiles 0-3,
      // group 1 d tiles 4-7. Each group passes the other half of its O and its (m, l, rounded
      // sum) through its own K area and a slice of the Q area, which the key loop no longer
      // reads, so one barrier suffices; both then take m = max(m0, m1) and add the two parts
      // scaled by 2^(m_g - m), and store their own half.
      const uint32_t dyn0 = lds_base - grp * L::GROUP_BYTES;  // start of the dynamic area
      LDS v4f* give = lds_at<v4f>(lds_base + L::OFF_K) + wave * 8 * 64 + lane;
      LDS v4f* take = lds_at<v4f>(dyn0 + (1 - grp) * L::GROUP_BYTES + L::OFF_K) + wave * 8 * 64 + lane;
      LDS v4f* xgive = lds_at<v4f>(dyn0 + L::OFF_Q + grp * 8192) + wave * 2 * 64 + lane;
      LDS v4f* xtake = lds_at<v4f>(dyn0 + L::OFF_Q + (1 - grp) * 8192) + wave * 2 * 64 + lane;
      if (grp == 0)
        give_half<4>(give);
      else
        give_half<0>(give);
      xgive[0] = v4f{m_run[0], m_run[1], l_run[0], l_run[1]};
      xgive[64] = v4f{o_sum[0][0], o_sum[1][0], 0.0f, 0.0f};
      __syncthreads();
      if (grp == 0) {
        merge_half<0>(take, xtake[0], xtake[64]);
        epilogue_staged<0>(vd, true);
      } else {
        merge_half<1>(take, xtake[0], xtake[64]);
        epilogue_staged<4>(vd, false);
      }
      return true;
    }
    if (G == 2 && grp == 1) return true;  // no key block: group 0 writes zeros and -inf
    if constexpr (G == 1) {
      wait_vm_all();
      __syncthreads();  // every wave's last V reads are done: V object 0 becomes the stage
      epilogue_staged_rows(vd);
    } else {
      epilogue<0, 8>(vd, true);
    }
    return true;
  }
};

// A tile on the BF16 score path, in a function of its own so that the two-group kernel's FP8
// path (256 registers per wave) is register-allocated without it: sharing one allocation costs
// the FP8 path spills around its loops. Only tiles that fail the precision guard make the call
// (which also saves the registers the calling convention asks the callee to preserve).
template <bool MX, bool FP8V, bool VMX>
__device__ __attribute__((noinline)) void slow_tile(const AttnParams* pp, uint8_t* smem, LDS uint8_t* va,
                                                    LDS uint8_t* vb, int grp, int seq, int head, int qtile) {
  // arguments arrive in vector registers: the uniform ones go back to scalar registers
  const uint64_t pa = (uint64_t)(uintptr_t)pp;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)pa);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(pa >> 32));
  const AttnParams& p = *reinterpret_cast<const AttnParams*>((uintptr_t)(((uint64_t)hi << 32) | lo));
  Attn<MX, FP8V, VMX> a(p, smem, __builtin_amdgcn_readfirstlane(grp), va, vb);
  a.seq = __builtin_amdgcn_readfirstlane(seq);
  a.head = __builtin_amdgcn_readfirstlane(head);
  a.load_meta();
  a.template run<1>(__builtin_amdgcn_readfirstlane(qtile));
}

template <bool MX, bool FP8V, bool VMX, bool QB>
__global__ __launch_bounds__(256 * Groups<FP8V>::G) void attn_fwd_kernel(AttnParams p) {
  extern __shared__ __align__(16) uint8_t smem[];
  int seq, head, qtile;
  if (p.tile_order != nullptr) {
    if ((int)blockIdx.x >= p.num_tiles) return;
    seq = p.tile_order[3 * blockIdx.x];
    head = p.tile_order[3 * blockIdx.x + 1];
    qtile = p.tile_order[3 * blockIdx.x + 2];
  } else if ((p.num_heads & 7) == 0) {
    // head h on XCD h % 8 (workgroup ids are dealt round-robin over the 8 XCDs): the XCD whose
    // workgroups quantized that head's Q and K and cast its V (their groups enumerate heads
    // fastest), so the codes they just wrote are in that XCD's L2; the XCD's tiles in (sequence,
    // head, tile) order. The grid is exactly num_seqs * num_heads * q_tiles.
    const int x = (int)(blockIdx.x & 7), k = (int)(blockIdx.x >> 3);
    qtile = k % p.q_tiles;
    const int rest = k / p.q_tiles, hx = p.num_heads >> 3;
    head = x + 8 * (rest % hx);
    seq = rest / hx;
    if (seq >= p.num_seqs) return;
  } else {
    const int per_xcd = (int)(gridDim.x >> 3);  // grid is a multiple of 8
    const int logical = (int)(blockIdx.x & 7) * per_xcd + (int)(blockIdx.x >> 3);
    if (logical >= p.num_tiles) return;
    qtile = logical % p.q_tiles;
    const int rest = logical / p.q_tiles;
    head = rest % p.num_heads;
    seq = rest / p.num_heads;
  }
  __shared__ __attribute__((aligned(16))) uint8_t va[Lay<FP8V, QB>::VOBJ_BYTES];
  __shared__ __attribute__((aligned(16))) uint8_t vb[Lay<FP8V, QB>::VOBJ_BYTES];
  const int grp = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 8));
  Attn<MX, FP8V, VMX, QB> a(p, smem, grp, LDS_PTR(uint8_t, va), LDS_PTR(uint8_t, vb));
  a.seq = seq;
  a.head = head;
  a.load_meta();
  if (qtile * BM >= a.Lq) return;
  if constexpr (Groups<FP8V>::G == 1 && !(MX && !QB)) {
    a.template run<2>(qtile);  // 512 registers per wave: both score loops fit in one allocation
  } else if constexpr (Groups<FP8V>::G == 1) {
    // BF16 V with MX Q/K: a tile that fails the guard runs the DQ pipeline (K dequantized once per
    // block into BF16 LDS tiles, Q into BF16 registers), inline: 512 registers hold both paths
    if (p.k_deq != nullptr) {
      // K's BF16 values come from the quantizer, a sign that the data is expected to fail the
      // guard: the DQ pipeline (K loaded like BF16 K) starts at once and takes the decision in its
      // prologue; a tile that may take FP8 scores then runs the FP8 path.
      Attn<MX, false, false, false, true, true> d(p, smem, grp, LDS_PTR(uint8_t, va), LDS_PTR(uint8_t, vb));
      d.seq = seq;
      d.head = head;
      d.load_meta();
      if (!d.template run<3>(qtile)) {
        __syncthreads();  // every wave has read the decision before the FP8 path's LDS writes
        if (!a.template run<0>(qtile)) {  // the same bounds pass again: FP8 scores (kept total)
          __syncthreads();
          d.template run<1>(qtile);
        }
      }
    } else if (!a.template run<0>(qtile)) {
      // every wave has read the guard's decision before the BF16 K tiles (which cover the
      // reduction slots) are written
      __syncthreads();
      Attn<MX, false, false, false, true> d(p, smem, grp, LDS_PTR(uint8_t, va), LDS_PTR(uint8_t, vb));
      d.seq = seq;
      d.head = head;
      d.load_meta();
      d.template run<1>(qtile);
    }
  } else if (!a.template run<0>(qtile)) {
    // guard failed: the two-group kernel's BF16 score loop, in a function of its own
    // The parameters are the kernel's only argument: the callee reads them in place in the
    // kernel-argument segment (taking the address of p instead makes the kernel itself read its
    // fields differently, to the FP8 loop's cost). The host compilation pass has no such segment.
#if defined(__HIP_DEVICE_COMPILE__)
    const AttnParams* pp = reinterpret_cast<const AttnParams*>(__builtin_amdgcn_kernarg_segment_ptr());
#else
    const AttnParams* pp = nullptr;
#endif
    slow_tile<MX, FP8V, VMX>(pp, smem, LDS_PTR(uint8_t, va), LDS_PTR(uint8_t, vb), grp, seq, head, qtile);
  }
}

template <bool MX, bool FP8V, bool VMX, bool QB = false>
hipError_t launch_variant(const AttnParams& p, dim3 grid, hipStream_t s, hipEvent_t start, hipEvent_t stop) {
  // Raising the dynamic LDS limit is a per-kernel, per-device attribute: done once per device.
  static std::atomic<uint64_t> configured{0};
  // the BF16-V kernel with MX Q/K also runs guard-failing tiles on BF16 K tiles (DQ): room for both
  constexpr int b0 = Lay<FP8V, QB>::TOTAL, b1 = Lay<FP8V, true>::TOTAL;
  const int bytes = (MX && !FP8V && !QB && b1 > b0) ? b1 : b0;
  const dim3 block(256 * Groups<FP8V>::G);
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const uint64_t bit = dev < 64 ? (uint64_t(1) << dev) : 0;
  if (bit == 0 || !(configured.load(std::memory_order_acquire) & bit)) {
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(&attn_fwd_kernel<MX, FP8V, VMX, QB>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
    if (e != hipSuccess) return e;
    configured.fetch_or(bit, std::memory_order_acq_rel);
  }
  if (start == nullptr && stop == nullptr) {
    hipLaunchKernelGGL((attn_fwd_kernel<MX, FP8V, VMX, QB>), grid, block, bytes, s, p);
    return hipGetLastError();
  }
  // The dispatch itself stamps the events: their interval is the kernel, without launch gaps.
  AttnParams arg = p;
  void* args[] = {&arg};
  return hipExtLaunchKernel(reinterpret_cast<const void*>(&attn_fwd_kernel<MX, FP8V, VMX, QB>), grid, block, args,
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
  if (p.qk_bf16) return launch_variant<false, false, false, true>(p, dim3(grid), s, start, stop);  // BF16 V checked
  if (pv_mode == LPFA_PV_MX) return launch_variant<true, true, true>(p, dim3(grid), s, start, stop);  // MX Q/K checked
  if (mx && fp8v) return launch_variant<true, true, false>(p, dim3(grid), s, start, stop);
  if (mx) return launch_variant<true, false, false>(p, dim3(grid), s, start, stop);
  if (fp8v) return launch_variant<false, true, false>(p, dim3(grid), s, start, stop);
  return launch_variant<false, false, false>(p, dim3(grid), s, start, stop);
}

}  // namespace lpfa
