// Measured ceilings for the roofline fractions that bench.py reports next to the published ones:
// dense FP8 and BF16 matrix-instruction rates, and HBM copy bandwidth, on the GPU at hand.
// A separate library (libpeak.so) built with the product library; it is not part of the C ABI in
// include/lpfa.h. Each launcher runs one kernel on the caller's stream and returns the hipError_t.
//
//   peak_mfma_fp8(waves_per_simd, iters, out, stream): every wave issues `iters` rounds of 8
//     independent v_mfma_scale_f32_16x16x128_f8f6f4 (65536 FLOP each, unit scales), the
//     instruction of the attention's FP8 score and P V products, on register operands.
//   peak_mfma_bf16(waves_per_simd, iters, out, stream): the same with v_mfma_f32_16x16x32_bf16
//     (16384 FLOP each), the instruction of the BF16 paths.
//   peak_copy(src, dst, bytes, stream): dst = src (bytes a multiple of 16), one 16-byte
//     nontemporal load and store per thread, one workgroup per 4 KiB; moves 2 * bytes through HBM.
//     Measured on 1 GiB: 6.6 TB/s, against 4.7-4.8 TB/s for a grid-stride loop of 4096 workgroups
//     with 8 chunks in flight per thread, and 5.1-5.7 TB/s for 2 or 4 chunks per thread.
// The matrix kernels launch 256 CUs x 4 SIMDs x waves_per_simd waves; `out` (one float per wave,
// device memory) receives a sum of the accumulators so the work cannot be dropped.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

constexpr int NUM_CU = 256;

__global__ __launch_bounds__(256) void mfma_fp8_kernel(int iters, float* out) {
  const int lane = threadIdx.x & 63;
  v8i a, b;
  for (int i = 0; i < 8; ++i) {
    a[i] = 0x38383838 ^ (lane & 1);  // E4M3 values near 1.0
    b[i] = 0x38383838 ^ (i & 1);
  }
  v4f acc[8];
  for (int c = 0; c < 8; ++c) acc[c] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[c] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, acc[c], 0, 0, 0, 127, 0, 127);
  }
  float s = 0.0f;
  for (int c = 0; c < 8; ++c) s += acc[c][0] + acc[c][1] + acc[c][2] + acc[c][3];
  if (lane == 0) out[blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6)] = s;
}

__global__ __launch_bounds__(256) void mfma_bf16_kernel(int iters, float* out) {
  const int lane = threadIdx.x & 63;
  v8bf a, b;
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(1.0f + 0.0078125f * (lane & 3));
    b[i] = (__bf16)(1.0f - 0.0078125f * (i & 1));
  }
  v4f acc[8];
  for (int c = 0; c < 8; ++c) acc[c] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[c], 0, 0, 0);
  }
  float s = 0.0f;
  for (int c = 0; c < 8; ++c) s += acc[c][0] + acc[c][1] + acc[c][2] + acc[c][3];
  if (lane == 0) out[blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6)] = s;
}

// One 16-byte chunk per thread: a grid of bytes / 4096 workgroups keeps every CU's queue of
// workgroups full until the end.
typedef unsigned v4u __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void copy_kernel(const v4u* __restrict__ src, v4u* __restrict__ dst, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
}

}  // namespace

extern "C" {

// One workgroup of 4 waves per CU and SIMD slot: waves_per_simd workgroups per CU.
int peak_mfma_fp8(int waves_per_simd, int iters, float* out, void* stream) {
  hipLaunchKernelGGL(mfma_fp8_kernel, dim3(NUM_CU * waves_per_simd), dim3(256), 0, static_cast<hipStream_t>(stream),
                     iters, out);
  return (int)hipGetLastError();
}

int peak_mfma_bf16(int waves_per_simd, int iters, float* out, void* stream) {
  hipLaunchKernelGGL(mfma_bf16_kernel, dim3(NUM_CU * waves_per_simd), dim3(256), 0, static_cast<hipStream_t>(stream),
                     iters, out);
  return (int)hipGetLastError();
}

// bytes must be a multiple of 16; src and dst 16-byte aligned.
int peak_copy(const void* src, void* dst, int64_t bytes, void* stream) {
  const int64_t n = bytes / 16, blocks = (n + 255) / 256;
  if (bytes % 16 != 0 || blocks > 0x7FFFFFFF) return (int)hipErrorInvalidValue;
  if (blocks == 0) return (int)hipSuccess;
  hipLaunchKernelGGL(copy_kernel, dim3((unsigned)blocks), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<const v4u*>(src), static_cast<v4u*>(dst), n);
  return (int)hipGetLastError();
}

}  // extern "C"
