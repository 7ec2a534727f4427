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
//   cube_mean   one wavefront per (b, h, cube): fp32 mean over valid rows;
//   block_score 32x32 tiles of the fp32 score matrix per (b, h) on the
//               fp32 matrix cores;
//   topk_rows   one wavefront per score row: exact k-th largest key by a
//               32-step bitwise search over order-preserving uint32 keys,
//               then an index-ordered compaction with ballots (no atomics,
//               deterministic).
#include "common.h"

namespace vsa {

namespace {

// Mean of each cube over its valid rows: xc [B, H, Np, D] bf16 -> [B, H, Nc, D] fp32.
// One wavefront per (b, h, cube), four cubes per workgroup.  Lane L reads the
// 16-byte chunk L % (D/8) of rows L / (D/8), + 64/(D/8), ... (fully coalesced
// 1 KB per instruction), keeps 8 fp32 partial sums, and the row groups are
// folded with cross-lane exchanges.
template <int D>
__global__ void __launch_bounds__(256) cube_mean(const uint16_t* __restrict__ xc, float* __restrict__ mean,
                                                 KGeom g, long long ncubes_total) {
  constexpr int CH = D / 8;         // lanes per row
  constexpr int RPI = 64 / CH;      // rows per load
  const long long cube_id = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (cube_id >= ncubes_total) return;  // whole wavefront leaves together
  const int lane = threadIdx.x & 63;
  const int c = (int)(cube_id % g.nc);
  int ct, cy, cx;
  cube_coords(g, c, ct, cy, cx);
  const uint4* base = reinterpret_cast<const uint4*>(xc + cube_id * 64 * D);
  float acc[8] = {};
#pragma unroll
  for (int it = 0; it < 64 / RPI; ++it) {
    const int row = it * RPI + lane / CH;
    const uint4 v = base[it * 64 + lane];
    if (local_valid(g, ct, cy, cx, row)) {
      const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc[2 * e] += __uint_as_float(w4[e] << 16);
        acc[2 * e + 1] += __uint_as_float(w4[e] & 0xFFFF0000u);
      }
    }
  }
#pragma unroll
  for (int off = CH; off < 64; off *= 2)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] += __shfl_xor(acc[e], off);
  if (lane < CH) {
    const float inv_n = 1.f / (float)cube_count(g, ct, cy, cx);
    float4* dst = reinterpret_cast<float4*>(mean + cube_id * D + lane * 8);
    dst[0] = make_float4(acc[0] * inv_n, acc[1] * inv_n, acc[2] * inv_n, acc[3] * inv_n);
    dst[1] = make_float4(acc[4] * inv_n, acc[5] * inv_n, acc[6] * inv_n, acc[7] * inv_n);
  }
}

// scores[bh, i, j] = sum_d qbar[bh, i, d] * kbar[bh, j, d] in fp32 on the
// matrix cores (v_mfma_f32_32x32x2_f32: fp32 products are exact, sums are
// fp32).  One wavefront per 32 x 32 output tile.  The contraction order over
// d is permuted identically for both operands so that each lane reads four
// consecutive floats: MFMA u of group t takes d = 8t + 4 h + u on lane half h.
template <int D>
__global__ void __launch_bounds__(64) block_score(const float* __restrict__ qbar, const float* __restrict__ kbar,
                                                  float* __restrict__ scores, int nc) {
  const long long bh = blockIdx.z;
  const int i0 = blockIdx.y * 32, j0 = blockIdx.x * 32;
  const int lane = threadIdx.x, h = lane >> 5, m = lane & 31;
  const float* qrow = qbar + (bh * nc + min(i0 + m, nc - 1)) * D;
  const float* krow = kbar + (bh * nc + min(j0 + m, nc - 1)) * D;
  const bool qin = i0 + m < nc, kin = j0 + m < nc;
  f32x16 acc = f32x16{};
  // All operand loads are issued before the first product (fully unrolled).
  float4 av[D / 8], bv[D / 8];
#pragma unroll
  for (int t = 0; t < D / 8; ++t) {
    av[t] = *reinterpret_cast<const float4*>(qrow + 8 * t + 4 * h);
    bv[t] = *reinterpret_cast<const float4*>(krow + 8 * t + 4 * h);
  }
#pragma unroll
  for (int t = 0; t < D / 8; ++t) {
    const float4 a = qin ? av[t] : make_float4(0.f, 0.f, 0.f, 0.f);
    const float4 b = kin ? bv[t] : make_float4(0.f, 0.f, 0.f, 0.f);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a.x, b.x, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a.y, b.y, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a.z, b.z, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a.w, b.w, acc, 0, 0, 0);
  }
  // acc[r]: row i0 + 8 (r/4) + 4 h + r%4, column j0 + m.
  const int j = j0 + m;
  if (j < nc) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int i = i0 + 8 * (r >> 2) + 4 * h + (r & 3);
      if (i < nc) scores[(bh * nc + i) * nc + j] = acc[r];
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

hipError_t launch_select_pooled(const KGeom& g, const float* qbar, const float* kbar, int topk, int32_t* idx,
                                float* scores, hipStream_t s);

hipError_t launch_select(const KGeom& g, const uint16_t* qc, const uint16_t* kc, int topk, int32_t* idx,
                         void* ws, hipStream_t s) {
  const size_t bh = (size_t)g.B * g.H;
  float* qbar = static_cast<float*>(ws);
  float* kbar = qbar + bh * g.nc * g.D;
  float* scores = kbar + bh * g.nc * g.D;
  const long long ncubes_total = (long long)bh * g.nc;
  const dim3 pg((unsigned)((ncubes_total + 3) / 4));
  if (g.D == 64) {
    hipLaunchKernelGGL(cube_mean<64>, pg, dim3(256), 0, s, qc, qbar, g, ncubes_total);
    hipLaunchKernelGGL(cube_mean<64>, pg, dim3(256), 0, s, kc, kbar, g, ncubes_total);
  } else {
    hipLaunchKernelGGL(cube_mean<128>, pg, dim3(256), 0, s, qc, qbar, g, ncubes_total);
    hipLaunchKernelGGL(cube_mean<128>, pg, dim3(256), 0, s, kc, kbar, g, ncubes_total);
  }
  return launch_select_pooled(g, qbar, kbar, topk, idx, scores, s);
}

size_t select_pooled_workspace_bytes(const KGeom& g) {
  return (size_t)g.B * g.H * g.nc * (size_t)g.nc * sizeof(float);
}

hipError_t launch_select_pooled(const KGeom& g, const float* qbar, const float* kbar, int topk, int32_t* idx,
                                float* scores, hipStream_t s) {
  const size_t bh = (size_t)g.B * g.H;
  const int tiles = (g.nc + 31) / 32;
  if (g.D == 64)
    hipLaunchKernelGGL(block_score<64>, dim3(tiles, tiles, (unsigned)bh), dim3(64), 0, s, qbar, kbar, scores, g.nc);
  else
    hipLaunchKernelGGL(block_score<128>, dim3(tiles, tiles, (unsigned)bh), dim3(64), 0, s, qbar, kbar, scores, g.nc);
  const long long nrows = (long long)bh * g.nc;
  const int per_lane = (g.nc + 63) / 64;
  // Every keys-per-lane count up to 8 has its own instantiation, larger ones
  // come in steps of a quarter to a half (the 32-step search costs one ballot
  // per key slot).
  if (per_lane <= 1)
    launch_topk<1>(scores, idx, nrows, g.nc, topk, s);
  else if (per_lane <= 2)
    launch_topk<2>(scores, idx, nrows, g.nc, topk, s);
  else if (per_lane <= 3)
    launch_topk<3>(scores, idx, nrows, g.nc, topk, s);
  else if (per_lane <= 4)
    launch_topk<4>(scores, idx, nrows, g.nc, topk, s);
  else if (per_lane <= 5)
    launch_topk<5>(scores, idx, nrows, g.nc, topk, s);
  else if (per_lane <= 6)
    launch_topk<6>(scores, idx, nrows, g.nc, topk, s);
  else if (per_lane <= 7)
    launch_topk<7>(scores, idx, nrows, g.nc, topk, s);
  else if (per_lane <= 8)
    launch_topk<8>(scores, idx, nrows, g.nc, topk, s);
  else if (per_lane <= 12)
    launch_topk<12>(scores, idx, nrows, g.nc, topk, s);
  else if (per_lane <= 16)
    launch_topk<16>(scores, idx, nrows, g.nc, topk, s);
  else if (per_lane <= 24)
    launch_topk<24>(scores, idx, nrows, g.nc, topk, s);
  else if (per_lane <= 32)
    launch_topk<32>(scores, idx, nrows, g.nc, topk, s);
  else if (per_lane <= 48)
    launch_topk<48>(scores, idx, nrows, g.nc, topk, s);
  else
    launch_topk<64>(scores, idx, nrows, g.nc, topk, s);
  return hipGetLastError();
}

}  // namespace vsa
