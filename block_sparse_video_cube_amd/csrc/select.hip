// Coarse stage: cube mean-pooling, pooled block scores, per-row top-k.
//
// VSA picks the important attention blocks dynamically and keeps about one
// minus the sparsity of them (FastVideo sparse-distillation article, section
// "2. 视频稀疏注意力VSA").  Convention: each cube is summarised by the mean of
// its valid tokens, a query cube scores a key cube by the dot product of the
// two means, and the k best key cubes are kept, equal scores going to the
// lower cube index, listed in ascending order.
//
// Three kernels:
//   cube_mean   one workgroup per (b, h, cube): fp32 mean over valid rows;
//   block_score 64x64 tiles of the fp32 score matrix per (b, h);
//   topk_rows   one wavefront per score row: exact k-th largest key by a
//               32-step bitwise search over order-preserving uint32 keys,
//               then an index-ordered compaction with ballots (no atomics,
//               deterministic).
#include "common.h"

namespace vsa {

namespace {

// Mean of each cube over its valid rows: qc [B, H, Np, D] bf16 -> [B, H, Nc, D] fp32.
template <int D>
__global__ void __launch_bounds__(256) cube_mean(const uint16_t* __restrict__ xc, float* __restrict__ mean,
                                                 KGeom g) {
  constexpr int RG = 256 / D;  // row groups
  __shared__ float part[RG][D];
  const int c = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  int ct, cy, cx;
  cube_coords(g, c, ct, cy, cx);
  const int d = threadIdx.x % D, rg = threadIdx.x / D;
  const uint16_t* base = xc + (((long long)b * g.H + h) * g.Np + 64LL * c) * D;
  float acc = 0.f;
  for (int l = rg; l < 64; l += RG) {
    if (local_valid(g, ct, cy, cx, l)) acc += bf16_to_f32(base[l * D + d]);
  }
  part[rg][d] = acc;
  __syncthreads();
  if (rg == 0) {
    float s = part[0][d];
#pragma unroll
    for (int r = 1; r < RG; ++r) s += part[r][d];
    const float n = (float)cube_count(g, ct, cy, cx);
    mean[(((long long)b * g.H + h) * g.nc + c) * D + d] = s / n;
  }
}

// scores[bh, i, j] = sum_d qbar[bh, i, d] * kbar[bh, j, d]  (fp32).
// 64x64 output tile per workgroup, 256 threads x (4x4) outputs, D in chunks of 32.
__global__ void __launch_bounds__(256) block_score(const float* __restrict__ qbar, const float* __restrict__ kbar,
                                                   float* __restrict__ scores, int nc, int D) {
  __shared__ float qs[32][64 + 1];
  __shared__ float ks[32][64 + 1];
  const long long bh = blockIdx.z;
  const int i0 = blockIdx.y * 64, j0 = blockIdx.x * 64;
  const int tx = threadIdx.x % 16, ty = threadIdx.x / 16;
  const float* qb = qbar + bh * nc * D;
  const float* kb = kbar + bh * nc * D;
  float acc[4][4] = {};
  for (int d0 = 0; d0 < D; d0 += 32) {
    for (int f = threadIdx.x; f < 64 * 32; f += 256) {
      const int r = f / 32, dd = f % 32;
      qs[dd][r] = (i0 + r < nc) ? qb[(long long)(i0 + r) * D + d0 + dd] : 0.f;
      ks[dd][r] = (j0 + r < nc) ? kb[(long long)(j0 + r) * D + d0 + dd] : 0.f;
    }
    __syncthreads();
#pragma unroll 4
    for (int dd = 0; dd < 32; ++dd) {
      float a[4], bb[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        a[u] = qs[dd][ty * 4 + u];
        bb[u] = ks[dd][tx * 4 + u];
      }
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[u][v] = fmaf(a[u], bb[v], acc[u][v]);
    }
    __syncthreads();
  }
  for (int u = 0; u < 4; ++u) {
    const int i = i0 + ty * 4 + u;
    if (i >= nc) continue;
    for (int v = 0; v < 4; ++v) {
      const int j = j0 + tx * 4 + v;
      if (j < nc) scores[(bh * nc + i) * nc + j] = acc[u][v];
    }
  }
}

// Order-preserving key of an fp32 score: larger score -> larger unsigned key;
// -0 is folded onto +0 so that they tie.
__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ int ballot_count(bool p) { return __popcll(__ballot(p)); }

// One wavefront per score row; MAXV keys per lane (nc <= 64 * MAXV).
template <int MAXV>
__global__ void __launch_bounds__(256) topk_rows(const float* __restrict__ scores, int32_t* __restrict__ idx,
                                                 long long nrows, int nc, int k) {
  const int lane = threadIdx.x & 63;
  const long long row = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= nrows) return;  // whole wavefront leaves together
  const float* sr = scores + row * nc;
  uint32_t key[MAXV];
#pragma unroll
  for (int v = 0; v < MAXV; ++v) {
    const int j = v * 64 + lane;
    key[v] = (j < nc) ? order_key(sr[j]) : 0u;
  }
  // Largest threshold t with count(key >= t) >= k: the k-th largest key.
  uint32_t thr = 0;
  for (int bit = 31; bit >= 0; --bit) {
    const uint32_t cand = thr | (1u << bit);
    int cnt = 0;
#pragma unroll
    for (int v = 0; v < MAXV; ++v) cnt += ballot_count(v * 64 + lane < nc && key[v] >= cand);
    if (cnt >= k) thr = cand;
  }
  int gt = 0;
#pragma unroll
  for (int v = 0; v < MAXV; ++v) gt += ballot_count(v * 64 + lane < nc && key[v] > thr);
  const int need_eq = k - gt;  // >= 1
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  int base = 0, eq_seen = 0;
  int32_t* out = idx + row * k;
#pragma unroll
  for (int v = 0; v < MAXV; ++v) {
    const int j = v * 64 + lane;
    const bool in = j < nc;
    const bool is_gt = in && key[v] > thr;
    const bool is_eq = in && key[v] == thr;
    const uint64_t eqm = __ballot(is_eq);
    const int eq_rank = eq_seen + __popcll(eqm & lt_mask);
    const bool sel = is_gt || (is_eq && eq_rank < need_eq);
    const uint64_t selm = __ballot(sel);
    if (sel) out[base + __popcll(selm & lt_mask)] = j;
    base += __popcll(selm);
    eq_seen += __popcll(eqm);
  }
}

template <int MAXV>
void launch_topk(const float* s, int32_t* idx, long long nrows, int nc, int k, hipStream_t st) {
  const unsigned blocks = (unsigned)((nrows + 3) / 4);
  hipLaunchKernelGGL(topk_rows<MAXV>, dim3(blocks), dim3(256), 0, st, s, idx, nrows, nc, k);
}

}  // namespace

size_t select_workspace_bytes(const KGeom& g) {
  const size_t bh = (size_t)g.B * g.H;
  const size_t means = 2 * bh * g.nc * g.D * sizeof(float);
  const size_t scores = bh * g.nc * (size_t)g.nc * sizeof(float);
  return means + scores;
}

hipError_t launch_select(const KGeom& g, const uint16_t* qc, const uint16_t* kc, int topk, int32_t* idx,
                         void* ws, hipStream_t s) {
  const size_t bh = (size_t)g.B * g.H;
  float* qbar = static_cast<float*>(ws);
  float* kbar = qbar + bh * g.nc * g.D;
  float* scores = kbar + bh * g.nc * g.D;
  const dim3 pg(g.nc, g.H, g.B);
  if (g.D == 64) {
    hipLaunchKernelGGL(cube_mean<64>, pg, dim3(256), 0, s, qc, qbar, g);
    hipLaunchKernelGGL(cube_mean<64>, pg, dim3(256), 0, s, kc, kbar, g);
  } else {
    hipLaunchKernelGGL(cube_mean<128>, pg, dim3(256), 0, s, qc, qbar, g);
    hipLaunchKernelGGL(cube_mean<128>, pg, dim3(256), 0, s, kc, kbar, g);
  }
  const int tiles = (g.nc + 63) / 64;
  hipLaunchKernelGGL(block_score, dim3(tiles, tiles, (unsigned)bh), dim3(256), 0, s, qbar, kbar, scores, g.nc,
                     g.D);
  const long long nrows = (long long)bh * g.nc;
  const int per_lane = (g.nc + 63) / 64;
  if (per_lane <= 1)
    launch_topk<1>(scores, idx, nrows, g.nc, topk, s);
  else if (per_lane <= 2)
    launch_topk<2>(scores, idx, nrows, g.nc, topk, s);
  else if (per_lane <= 4)
    launch_topk<4>(scores, idx, nrows, g.nc, topk, s);
  else if (per_lane <= 8)
    launch_topk<8>(scores, idx, nrows, g.nc, topk, s);
  else if (per_lane <= 16)
    launch_topk<16>(scores, idx, nrows, g.nc, topk, s);
  else if (per_lane <= 32)
    launch_topk<32>(scores, idx, nrows, g.nc, topk, s);
  else
    launch_topk<64>(scores, idx, nrows, g.nc, topk, s);
  return hipGetLastError();
}

}  // namespace vsa
