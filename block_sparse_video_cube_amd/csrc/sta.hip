// Sliding-tile block lists: the static alternative to the top-k selection.
//
// Sliding-tile attention (STA) is one of the attention backends the FastVideo
// attention-backend article lists (item "SLIDING_TILE_ATTN"; its figure
// compares NATTEN, Tiled NATTEN and STA, the last one free of partially
// masked blocks).  With 4x4x4 cubes as tiles, STA is the fine stage of this
// library fed a fixed block list: each query cube attends to a window of
// (wt, wh, ww) key cubes, centred on it where possible and shifted inwards at
// the grid borders so that every list has the same length
// k = min(wt, Ct) * min(wh, Ch) * min(ww, Cw).  Rows are ascending because the
// window is enumerated in raster order of cube coordinates.
#include "common.h"

namespace vsa {

namespace {

// First key-cube coordinate of the window along one axis.
__device__ __forceinline__ int window_start(int c, int n, int w) {
  if (w >= n) return 0;
  return min(max(c - (w - 1) / 2, 0), n - w);
}

// One thread per output entry (b, h, i, s), grid-stride.
__global__ void __launch_bounds__(256) sta_index_kernel(int32_t* __restrict__ idx, KGeom g, int wt, int wh, int ww,
                                                         int kt, int kh, int kw, long long total) {
  const int k = kt * kh * kw;
  for (long long e = blockIdx.x * 256LL + threadIdx.x; e < total; e += (long long)gridDim.x * 256) {
    const int s = (int)(e % k);
    const int i = (int)((e / k) % g.nc);
    int ct, cy, cx;
    cube_coords(g, i, ct, cy, cx);
    const int st = s / (kh * kw), sy = (s / kw) % kh, sx = s % kw;
    const int t0 = window_start(ct, g.ct, wt), y0 = window_start(cy, g.ch, wh), x0 = window_start(cx, g.cw, ww);
    idx[e] = ((t0 + st) * g.ch + (y0 + sy)) * g.cw + (x0 + sx);
  }
}

}  // namespace

hipError_t launch_sta_index(const KGeom& g, int wt, int wh, int ww, int32_t* idx, hipStream_t s) {
  const int kt = min(wt, g.ct), kh = min(wh, g.ch), kw = min(ww, g.cw);
  const long long total = (long long)g.B * g.H * g.nc * kt * kh * kw;
  const long long blocks = (total + 255) / 256;
  const unsigned grid = (unsigned)(blocks < (1LL << 20) ? blocks : (1LL << 20));
  hipLaunchKernelGGL(sta_index_kernel, dim3(grid), dim3(256), 0, s, idx, g, wt, wh, ww, kt, kh, kw, total);
  return hipGetLastError();
}

}  // namespace vsa
