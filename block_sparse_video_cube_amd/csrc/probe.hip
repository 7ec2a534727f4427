// Probes for the benchmark: the sustained rate of v_mfma_f32_32x32x16_bf16
// on this device and the shader clock while it runs, a measured second
// denominator beside the published bf16 peak; and the rates of plain HBM
// streams (copy, read, write), the same beside the published 8 TB/s.
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

// HBM streams over n 16-byte words, grid-stride, four words per thread per
// round (loads of a round issued before its stores).  KIND 0: dst = src;
// 1: read src (a checksum that is stored only if it equals an impossible
// value, so the loads stay); 2: write dst.  Stores bypass the caches'
// retention (nontemporal): they are not read back.
template <int KIND>
__global__ void __launch_bounds__(256) hbm_stream(const uint4* __restrict__ src, uint4* __restrict__ dst,
                                                  long long n) {
  constexpr int U = 4;
  const long long stride = (long long)gridDim.x * 256 * U;
  uint32_t acc = 0;
  for (long long base = (long long)blockIdx.x * 256 * U + threadIdx.x; base < n; base += stride) {
    uint4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const long long i = base + 256LL * u;
      if (KIND == 2) v[u] = make_uint4((uint32_t)i, (uint32_t)(i >> 32), 0u, 0u);
      else v[u] = i < n ? src[i] : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const long long i = base + 256LL * u;
      if (KIND == 1) {
        acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
      } else if (i < n) {
        typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
        __builtin_nontemporal_store(u32x4{v[u].x, v[u].y, v[u].z, v[u].w}, reinterpret_cast<u32x4*>(dst + i));
      }
    }
  }
  if (KIND == 1 && acc == 0x9E3779B9u && dst) dst[0] = make_uint4(acc, 0u, 0u, 0u);
}

}  // namespace

hipError_t launch_hbm_probe(int kind, const void* src, void* dst, long long words, hipStream_t s) {
  const dim3 grid(16384), block(256);
  const uint4* a = static_cast<const uint4*>(src);
  uint4* b = static_cast<uint4*>(dst);
  if (kind == 0) hipLaunchKernelGGL(hbm_stream<0>, grid, block, 0, s, a, b, words);
  else if (kind == 1) hipLaunchKernelGGL(hbm_stream<1>, grid, block, 0, s, a, b, words);
  else hipLaunchKernelGGL(hbm_stream<2>, grid, block, 0, s, a, b, words);
  return hipGetLastError();
}

hipError_t launch_mfma_probe(int blocks, int iters, float* sink, unsigned long long* clk, hipStream_t s) {
  hipLaunchKernelGGL(mfma_probe, dim3(blocks), dim3(256), 0, s, iters, sink, clk);
  return hipGetLastError();
}

}  // namespace vsa
