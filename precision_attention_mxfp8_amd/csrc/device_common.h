// Device-side helpers shared by the gfx950 kernels: vector types and the two hardware
// conversions the path relies on (float -> E4M3 pair, float -> BF16), both round to
// nearest even.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "lpfa.h"

namespace lpfa {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

// Two floats -> two E4M3 codes in the low 16 bits (first value in the low byte).
// The hardware conversion is OCP E4M3FN with round-to-nearest-even; magnitudes above
// 464 would become NaN, so callers clamp to +-448 first when the input can exceed it.
__device__ __forceinline__ uint32_t cvt_pk_e4m3(float a, float b) {
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false) & 0xFFFFu;
}

// Four floats -> four E4M3 codes packed little-endian in one word.
__device__ __forceinline__ uint32_t cvt4_e4m3(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  return (uint32_t)w;
}

// The same four codes written over a register's old contents: both halves are replaced, so the
// result does not depend on `old`, and no zeroing instruction precedes the first conversion.
__device__ __forceinline__ uint32_t cvt4_e4m3_over(uint32_t old, float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, (int)old, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  return (uint32_t)w;
}

__device__ __forceinline__ float clamp448(float x) { return fminf(fmaxf(x, -448.0f), 448.0f); }

// Two floats -> two BF16 (round to nearest even) packed in one word, first in the low half: one
// v_cvt_pk_bf16_f32 (element-wise casts would convert each value alone and then shift and merge).
typedef float cvt_f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 cvt_bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t cvt_pk_bf16(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(cvt_f32x2_t{a, b}, cvt_bf16x2_t));
}

// Four E4M3 codes (one word) times the power of two `scale` (only its exponent field is read, so
// an E8M0 byte b converts as __uint_as_float(b << 23), b = 0 as 2^-127) -> four BF16 in two words,
// with the hardware's scaled conversion. The quantizer's BF16 output of the quantized values and
// the attention's dequantization of K both use it, so the two agree bit for bit.
__device__ __forceinline__ uint2 fp8x4_scaled_bf16(uint32_t w, float scale) {
  return make_uint2(__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w, scale, false)),
                    __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w, scale, true)));
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Block exponent from the bits of amax (a non-negative float).
//   RCEIL: smallest e with amax <= 448 * 2^e. For amax = 1.m * 2^E (normal), 448 = 1.75 * 2^8,
//          so e = E - 8 if 1.m <= 1.75 (mantissa field <= 0x600000), else E - 7.
//   FLOOR: e = floor(log2 amax) - 8 = E - 8.
// Zero or subnormal amax gives an exponent below -127 under both rules: clamp to -127.
__device__ __forceinline__ int block_exponent(float amax, int mode) {
  uint32_t bits = __float_as_uint(amax);
  int biased = (int)(bits >> 23);
  uint32_t mant = bits & 0x7FFFFFu;
  int e = biased - 135;
  if (mode == LPFA_SCALING_RCEIL && mant > 0x600000u) e += 1;
  if (biased == 0) e = -127;
  return e < -127 ? -127 : e;  // the largest finite amax gives e = 120, so no upper clamp is hit
}

}  // namespace lpfa
