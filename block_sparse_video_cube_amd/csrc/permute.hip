// Cube permutation kernels: raster tokens <-> cube-major rows.
//
// Grouping the latent grid into whole 4x4x4 cubes is what lets every attention
// block be kept or skipped as a unit, with no partially masked ("mixed")
// blocks (FastVideo sparse-distillation article, figure comparing attention
// patterns in section "2. 视频稀疏注意力VSA"; FastVideo attention-backend
// article, figure on NATTEN / Tiled NATTEN / STA).
//
// These kernels only move bits (HBM bound).  One workgroup moves one
// (batch, head, cube) tile of 64 rows x D: reads are 16-byte chunks of token
// rows, writes are one contiguous tile.
#include "common.h"

namespace vsa {

namespace {

constexpr int kThreads = 256;

// The 16-byte chunks f = threadIdx.x + 256 it (it < IT) of one cube's 64 rows
// of head h, read from the raster rows: all loads are issued before any is
// used.  ok[it]: the chunk's token is valid (else val[it] = 0).  Chunk f is
// chunk f % (D/8) of local token f / (D/8).
template <int D, int IT>
__device__ __forceinline__ void gather_cube(const uint16_t* __restrict__ x, const KGeom& g, int b, int h, int ct,
                                            int cy, int cx, uint4 (&val)[IT], bool (&ok)[IT]) {
  constexpr int CH = D / 8;
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const int f = threadIdx.x + kThreads * it;
    const int l = f / CH, ch = f % CH;
    const int t = 4 * ct + (l >> 4), y = 4 * cy + ((l >> 2) & 3), xx = 4 * cx + (l & 3);
    ok[it] = t < g.T && y < g.Hg && xx < g.W;
    const long long s = ((long long)t * g.Hg + y) * g.W + xx;
    val[it] = ok[it] ? reinterpret_cast<const uint4*>(x + (((long long)b * g.S + s) * g.H + h) * D)[ch]
                     : make_uint4(0, 0, 0, 0);
  }
}

// [B, S, H, D] -> [B, H, Np, D]; padded rows become zero.  COMPACT: local
// token l goes to row compact_row(l) of its cube (valid tokens first).
template <int D, bool COMPACT>
__global__ void __launch_bounds__(kThreads) permute_token_major(const uint16_t* __restrict__ x,
                                                                uint16_t* __restrict__ xc, KGeom g) {
  constexpr int CH = D / 8;  // 16-byte chunks per row
  const int c = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  int ct, cy, cx;
  cube_coords(g, c, ct, cy, cx);
  uint4* out = reinterpret_cast<uint4*>(xc + (((long long)b * g.H + h) * g.Np + 64LL * c) * D);
  // (Issuing every load first, as the kernels below do, measured 1 % slower
  // here: each chunk goes straight back out.)
  for (int f = threadIdx.x; f < 64 * CH; f += kThreads) {
    const int l = f / CH, ch = f % CH;
    const int t = 4 * ct + (l >> 4), y = 4 * cy + ((l >> 2) & 3), xx = 4 * cx + (l & 3);
    uint4 val = make_uint4(0, 0, 0, 0);
    if (t < g.T && y < g.Hg && xx < g.W) {
      const long long s = ((long long)t * g.Hg + y) * g.W + xx;
      val = reinterpret_cast<const uint4*>(x + (((long long)b * g.S + s) * g.H + h) * D)[ch];
    }
    out[COMPACT ? compact_row(g, ct, cy, cx, l) * CH + ch : f] = val;
  }
}

// [B, S, H, D] -> [B, H, Np, D] as permute_token_major, and in the same pass
// the fp32 mean of every cube over its valid tokens -> mean [B, H, Nc, D].
// Thread t always handles 16-byte chunk t % (D/8) of its rows, so it keeps 8
// partial sums; threads with equal chunk are folded by cross-lane exchanges
// inside a wavefront and through LDS across the four wavefronts.
//
// With WRITE = false only the means are produced (the fine stage can gather
// raster-order rows itself, so the cube-major copy is not needed).  COMPACT:
// the copy is in compact order (rows as permute_token_major<D, true>); the
// sums are the same, in the same order.
template <int D, bool WRITE, bool COMPACT>
__global__ void __launch_bounds__(kThreads) permute_pool(const uint16_t* __restrict__ x, uint16_t* __restrict__ xc,
                                                         float* __restrict__ mean, KGeom g) {
  constexpr int CH = D / 8;
  __shared__ float part[kThreads / 64][D];
  const int c = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  int ct, cy, cx;
  cube_coords(g, c, ct, cy, cx);
  const long long cube_row = ((long long)b * g.H + h) * g.Np + 64LL * c;
  uint4* out = WRITE ? reinterpret_cast<uint4*>(xc + cube_row * D) : nullptr;
  float acc[8] = {};
  constexpr int IT = 64 * CH / kThreads;
  uint4 val[IT];
  bool ok[IT];
  gather_cube<D, IT>(x, g, b, h, ct, cy, cx, val, ok);
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const int f = threadIdx.x + kThreads * it;
    if (ok[it]) {  // padded tokens add nothing (not even a +0 to a -0 sum)
      const uint32_t w4[4] = {val[it].x, val[it].y, val[it].z, val[it].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc[2 * e] += __uint_as_float(w4[e] << 16);
        acc[2 * e + 1] += __uint_as_float(w4[e] & 0xFFFF0000u);
      }
    }
    if (WRITE) out[COMPACT ? compact_row(g, ct, cy, cx, f / CH) * CH + f % CH : f] = val[it];
  }
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
  for (int off = CH; off < 64; off *= 2)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] += __shfl_xor(acc[e], off);
  if (lane < CH) {
#pragma unroll
    for (int e = 0; e < 8; ++e) part[w][lane * 8 + e] = acc[e];
  }
  __syncthreads();
  if (threadIdx.x < D) {
    float sum = 0.f;
#pragma unroll
    for (int r = 0; r < kThreads / 64; ++r) sum += part[r][threadIdx.x];
    mean[(((long long)b * g.H + h) * g.nc + c) * D + threadIdx.x] = sum / (float)cube_count(g, ct, cy, cx);
  }
}

// [B, S, H, D] -> [B, H, Nc, D, 64]: each cube stored transposed (d-major).
template <int D>
__global__ void __launch_bounds__(kThreads) permute_dim_major(const uint16_t* __restrict__ x,
                                                              uint16_t* __restrict__ xc, KGeom g) {
  constexpr int CH = D / 8;
  constexpr int LD = D + 8;  // padded LDS row (halfwords), keeps 16-byte alignment
  __shared__ __attribute__((aligned(16))) uint16_t tile[64 * LD];
  const int c = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  int ct, cy, cx;
  cube_coords(g, c, ct, cy, cx);
  {
    constexpr int IT = 64 * CH / kThreads;
    uint4 val[IT];
    bool ok[IT];
    gather_cube<D, IT>(x, g, b, h, ct, cy, cx, val, ok);
#pragma unroll
    for (int it = 0; it < IT; ++it) {
      const int f = threadIdx.x + kThreads * it;
      *reinterpret_cast<uint4*>(tile + (f / CH) * LD + (f % CH) * 8) = val[it];
    }
  }
  __syncthreads();
  uint4* out = reinterpret_cast<uint4*>(xc + (((long long)b * g.H + h) * g.Np + 64LL * c) * D);
  for (int f = threadIdx.x; f < D * 8; f += kThreads) {
    const int d = f >> 3, lg = f & 7;
    uint32_t w[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t lo = tile[(8 * lg + 2 * e) * LD + d];
      const uint32_t hi = tile[(8 * lg + 2 * e + 1) * LD + d];
      w[e] = lo | (hi << 16);
    }
    out[f] = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

// [B, S, H, D] -> [B, H, Nc, 4, D, 16]: each cube in compact order, cut
// into four 16-row slots, each slot stored transposed (channel-major), so a
// slot is one contiguous D x 16 block.
template <int D>
__global__ void __launch_bounds__(kThreads) permute_slots(const uint16_t* __restrict__ x,
                                                          uint16_t* __restrict__ xs, KGeom g) {
  constexpr int CH = D / 8;
  constexpr int LD = D + 8;  // padded LDS row (halfwords), keeps 16-byte alignment
  __shared__ __attribute__((aligned(16))) uint16_t tile[64 * LD];
  const int c = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  int ct, cy, cx;
  cube_coords(g, c, ct, cy, cx);
  {
    constexpr int IT = 64 * CH / kThreads;
    uint4 val[IT];
    bool ok[IT];
    gather_cube<D, IT>(x, g, b, h, ct, cy, cx, val, ok);
#pragma unroll
    for (int it = 0; it < IT; ++it) {
      const int f = threadIdx.x + kThreads * it;
      *reinterpret_cast<uint4*>(tile + compact_row(g, ct, cy, cx, f / CH) * LD + (f % CH) * 8) = val[it];
    }
  }
  __syncthreads();
  // 16-byte chunk f of the output cube: slot f / (2 D), channel (f / 2) % D,
  // compact rows 16 slot + 8 (f % 2) .. + 7.
  uint4* out = reinterpret_cast<uint4*>(xs + (((long long)b * g.H + h) * g.Np + 64LL * c) * D);
  for (int f = threadIdx.x; f < D * 8; f += kThreads) {
    const int sl = f / (2 * D), d = (f >> 1) % D, r0 = 16 * sl + 8 * (f & 1);
    uint32_t w[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t lo = tile[(r0 + 2 * e) * LD + d];
      const uint32_t hi = tile[(r0 + 2 * e + 1) * LD + d];
      w[e] = lo | (hi << 16);
    }
    out[f] = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

// [B, H, Np, D] -> [B, S, H, D]; padded rows are dropped.
template <int D>
__global__ void __launch_bounds__(kThreads) unpermute_token_major(const uint16_t* __restrict__ xc,
                                                                  uint16_t* __restrict__ x, KGeom g) {
  constexpr int CH = D / 8;
  const int c = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  int ct, cy, cx;
  cube_coords(g, c, ct, cy, cx);
  const uint4* in = reinterpret_cast<const uint4*>(xc + (((long long)b * g.H + h) * g.Np + 64LL * c) * D);
  for (int f = threadIdx.x; f < 64 * CH; f += kThreads) {
    const int l = f / CH, ch = f % CH;
    const int t = 4 * ct + (l >> 4), y = 4 * cy + ((l >> 2) & 3), xx = 4 * cx + (l & 3);
    if (t < g.T && y < g.Hg && xx < g.W) {
      const long long s = ((long long)t * g.Hg + y) * g.W + xx;
      reinterpret_cast<uint4*>(x + (((long long)b * g.S + s) * g.H + h) * D)[ch] = in[f];
    }
  }
}

}  // namespace

template <int D>
void launch_permute_d(const KGeom& g, const uint16_t* x, uint16_t* xc, int layout, hipStream_t s) {
  const dim3 grid(g.nc, g.H, g.B);
  switch (layout) {
    case VSA_LAYOUT_TOKEN_MAJOR: permute_token_major<D, false><<<grid, dim3(kThreads), 0, s>>>(x, xc, g); break;
    case VSA_LAYOUT_TOKEN_COMPACT: permute_token_major<D, true><<<grid, dim3(kThreads), 0, s>>>(x, xc, g); break;
    case VSA_LAYOUT_DIM_SLOTS: permute_slots<D><<<grid, dim3(kThreads), 0, s>>>(x, xc, g); break;
    default: permute_dim_major<D><<<grid, dim3(kThreads), 0, s>>>(x, xc, g); break;
  }
}

hipError_t launch_permute(const KGeom& g, const uint16_t* x, uint16_t* xc, int layout, hipStream_t s) {
  if (g.D == 64) launch_permute_d<64>(g, x, xc, layout, s);
  else launch_permute_d<128>(g, x, xc, layout, s);
  return hipGetLastError();
}

template <int D>
void launch_permute_pool_d(const KGeom& g, const uint16_t* x, uint16_t* xc, float* mean, bool compact,
                           hipStream_t s) {
  const dim3 grid(g.nc, g.H, g.B);
  if (!xc) permute_pool<D, false, false><<<grid, dim3(kThreads), 0, s>>>(x, xc, mean, g);
  else if (compact) permute_pool<D, true, true><<<grid, dim3(kThreads), 0, s>>>(x, xc, mean, g);
  else permute_pool<D, true, false><<<grid, dim3(kThreads), 0, s>>>(x, xc, mean, g);
}

hipError_t launch_permute_pool(const KGeom& g, const uint16_t* x, uint16_t* xc, float* mean, bool compact,
                               hipStream_t s) {
  if (g.D == 64) launch_permute_pool_d<64>(g, x, xc, mean, compact, s);
  else launch_permute_pool_d<128>(g, x, xc, mean, compact, s);
  return hipGetLastError();
}

hipError_t launch_unpermute(const KGeom& g, const uint16_t* xc, uint16_t* x, hipStream_t s) {
  const dim3 grid(g.nc, g.H, g.B);
  if (g.D == 64)
    hipLaunchKernelGGL(unpermute_token_major<64>, grid, dim3(kThreads), 0, s, xc, x, g);
  else
    hipLaunchKernelGGL(unpermute_token_major<128>, grid, dim3(kThreads), 0, s, xc, x, g);
  return hipGetLastError();
}

}  // namespace vsa
