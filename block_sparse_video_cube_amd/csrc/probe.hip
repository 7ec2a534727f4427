// Matrix-core probe for the benchmark: the sustained rate of
// v_mfma_f32_32x32x16_bf16 on this device and the shader clock while it runs,
// a measured second denominator beside the published bf16 peak.
#include "common.h"

namespace vsa {

namespace {

// Every wavefront issues iters x 8 independent products on register operands
// (32768 flops each) and times its loop with the shader-clock counter
// (s_memtime) and the constant 100 MHz counter (s_memrealtime).
__global__ void __launch_bounds__(256, 2) mfma_probe(int iters, float* __restrict__ sink,
                                                     unsigned long long* __restrict__ clk) {
  const int lane = threadIdx.x & 63;
  bf16x8 a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = (__bf16)(0.001f * (float)((lane + e) & 7));
    b[e] = (__bf16)(0.001f * (float)((lane * 3 + e) & 7));
  }
  f32x16 acc[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) acc[k] = f32x16{};
  const unsigned long long t0 = __builtin_amdgcn_s_memtime(), r0 = __builtin_amdgcn_s_memrealtime();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int k = 0; k < 8; ++k) acc[k] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[k], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < 8; ++k)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[k][r];
  const unsigned long long t1 = __builtin_amdgcn_s_memtime(), r1 = __builtin_amdgcn_s_memrealtime();
  sink[blockIdx.x * 256 + threadIdx.x] = s;
  if (threadIdx.x == 0) {
    clk[2 * blockIdx.x] = t1 - t0;
    clk[2 * blockIdx.x + 1] = r1 - r0;
  }
}

}  // namespace

hipError_t launch_mfma_probe(int blocks, int iters, float* sink, unsigned long long* clk, hipStream_t s) {
  hipLaunchKernelGGL(mfma_probe, dim3(blocks), dim3(256), 0, s, iters, sink, clk);
  return hipGetLastError();
}

}  // namespace vsa
