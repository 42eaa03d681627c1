// Measurement probes: the ceilings the hot-path kernels are compared with, measured on the chip
// by kernels of this library instead of taken from the data sheet. Not part of the hot path.
//   * k_peak_mfma_bf16: back-to-back v_mfma_f32_32x32x16_bf16 from registers, four independent
//     accumulator chains per wavefront so each instruction issues as soon as the matrix core
//     takes it; 32768 flops per instruction.
//   * k_peak_copy: a streaming copy laid out like the cache writes (16 bytes per lane, two
//     vectors per thread, both loads issued before the first store).
#include "common.h"

namespace skv {

__global__ void __launch_bounds__(256) k_peak_mfma_bf16(float* out, int iters) {
  // operands depend on the lane, so the compiler cannot fold the products away
  bf16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (bf16_t)(0.001f * (float)((threadIdx.x + i) & 7));
    b[i] = (bf16_t)(0.002f * (float)((threadIdx.x * 3 + i) & 7));
  }
  f32x16 acc[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) acc[j] = f32x16{};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[j], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int e = 0; e < 16; ++e) s += acc[j][e];
  out[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
}

constexpr int kPeakCopyPer = 2;
__global__ void __launch_bounds__(256) k_peak_copy(const i32x4* __restrict__ src,
                                                   i32x4* __restrict__ dst, size_t n) {
  const size_t i0 = (size_t)blockIdx.x * (256 * kPeakCopyPer) + threadIdx.x;
  i32x4 r[kPeakCopyPer];
#pragma unroll
  for (int u = 0; u < kPeakCopyPer; ++u) {
    const size_t i = i0 + (size_t)u * 256;
    if (i < n) r[u] = __builtin_nontemporal_load(src + i);
  }
#pragma unroll
  for (int u = 0; u < kPeakCopyPer; ++u) {
    const size_t i = i0 + (size_t)u * 256;
    if (i < n) dst[i] = r[u];
  }
}

hipError_t launch_peak_mfma_bf16(float* out, int workgroups, int iters, hipStream_t s) {
  hipLaunchKernelGGL(k_peak_mfma_bf16, dim3((unsigned)workgroups), dim3(256), 0, s, out, iters);
  return hipGetLastError();
}

hipError_t launch_peak_copy(void* dst, const void* src, size_t bytes, hipStream_t s) {
  const size_t n = bytes / 16;
  const size_t blocks = (n + 256 * kPeakCopyPer - 1) / (256 * kPeakCopyPer);
  hipLaunchKernelGGL(k_peak_copy, dim3((unsigned)blocks), dim3(256), 0, s, (const i32x4*)src, (i32x4*)dst, n);
  return hipGetLastError();
}

}  // namespace skv
