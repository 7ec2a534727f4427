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
//               bitwise search over order-preserving uint32 keys (upper 16
//               bits over all keys, lower 16 over the keys of the threshold's
//               bucket), then an index-ordered compaction with ballots (no
//               atomics, deterministic).
#include "common.h"

namespace vsa {

namespace {

// Mean of each cube over its valid rows: xc [B, H, Np, D] bf16 -> [B, H, Nc, D] fp32.
// One wavefront per (b, h, cube), four cubes per workgroup.  The fp32 sums
// are taken in exactly the order of the pooling kernel that permute_pool
// runs on the raster rows (so both entry points of the coarse stage see the
// same means, bit for bit): that kernel's thread 64 w + L (w = 0..3) adds
// chunk L % (D/8) of rows (64 w + L) / (D/8) + 256 it / (D/8), it = 0, 1, ...
// in turn, folds its wavefront with cross-lane exchanges, and the four
// wavefront sums are added in order w = 0..3 and divided by the count.  Here
// lane L keeps those four partial sums itself.  Every load is a fully
// coalesced 1 KB (chunk 64 w + 256 it + L of the tile).
template <int D>
__global__ void __launch_bounds__(256) cube_mean(const uint16_t* __restrict__ xc, float* __restrict__ mean,
                                                 KGeom g, long long ncubes_total) {
  constexpr int CH = D / 8;         // lanes per row
  constexpr int IT = 64 * CH / 256; // rows per thread of the pooling kernel
  const long long cube_id = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (cube_id >= ncubes_total) return;  // whole wavefront leaves together
  const int lane = threadIdx.x & 63;
  const int c = (int)(cube_id % g.nc);
  int ct, cy, cx;
  cube_coords(g, c, ct, cy, cx);
  const uint4* base = reinterpret_cast<const uint4*>(xc + cube_id * 64 * D);
  float acc[4][8] = {};
#pragma unroll
  for (int w = 0; w < 4; ++w)
#pragma unroll
    for (int it = 0; it < IT; ++it) {
      const int f = 64 * w + 256 * it + lane;
      const uint4 v = base[f];
      if (local_valid(g, ct, cy, cx, f / CH)) {
        const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          acc[w][2 * e] += __uint_as_float(w4[e] << 16);
          acc[w][2 * e + 1] += __uint_as_float(w4[e] & 0xFFFF0000u);
        }
      }
    }
#pragma unroll
  for (int w = 0; w < 4; ++w)
#pragma unroll
    for (int off = CH; off < 64; off *= 2)
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[w][e] += __shfl_xor(acc[w][e], off);
  if (lane < CH) {
    const float n = (float)cube_count(g, ct, cy, cx);
    float r[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float sum = 0.f;
#pragma unroll
      for (int w = 0; w < 4; ++w) sum += acc[w][e];
      r[e] = sum / n;
    }
    float4* dst = reinterpret_cast<float4*>(mean + cube_id * D + lane * 8);
    dst[0] = make_float4(r[0], r[1], r[2], r[3]);
    dst[1] = make_float4(r[4], r[5], r[6], r[7]);
  }
}

// scores[bh, i, j] = sum_d qbar[bh, i, d] * kbar[bh, j, d] in fp32 on the
// matrix cores (v_mfma_f32_32x32x2_f32: fp32 products are exact, sums are
// fp32).  One wavefront per 32 x 64 output tile: two 32 x 32 accumulators
// share the Q operand, and their products alternate, so neither waits for
// its own previous product.  The contraction order over d is permuted
// identically for both operands so that each lane reads four consecutive
// floats: MFMA u of group t takes d = 8t + 4 h + u on lane half h (every
// output element sums its products in the same order as with one
// accumulator).  Operands are loaded a half of D at a time.
// Placement: the tiles of all heads, head by head and row by row, are cut
// into 8 contiguous ranges, one per XCD (workgroup w runs on XCD w mod 8), so
// each XCD works through whole heads in turn and their means stay in its L2.
template <int D>
__global__ void __launch_bounds__(64) block_score(const float* __restrict__ qbar, const float* __restrict__ kbar,
                                                  float* __restrict__ scores, int nc, int ti, int tj,
                                                  long long per_xcd, long long units) {
  const long long u = (blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
  if (u >= units) return;
  const int per_head = ti * tj;
  const long long bh = u / per_head;
  const int t = (int)(u - bh * per_head);
  const int i0 = (t / tj) * 32, j0 = (t % tj) * 64;
  const int lane = threadIdx.x, h = lane >> 5, m = lane & 31;
  const float* qrow = qbar + (bh * nc + min(i0 + m, nc - 1)) * D;
  const float* krow0 = kbar + (bh * nc + min(j0 + m, nc - 1)) * D;
  const float* krow1 = kbar + (bh * nc + min(j0 + 32 + m, nc - 1)) * D;
  const bool qin = i0 + m < nc, kin0 = j0 + m < nc, kin1 = j0 + 32 + m < nc;
  f32x16 acc0 = f32x16{}, acc1 = f32x16{};
  constexpr int TH = D / 16;  // groups of 8 d per half
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    float4 av[TH], bv0[TH], bv1[TH];
#pragma unroll
    for (int tt = 0; tt < TH; ++tt) {
      const int d = 8 * (half * TH + tt) + 4 * h;
      av[tt] = *reinterpret_cast<const float4*>(qrow + d);
      bv0[tt] = *reinterpret_cast<const float4*>(krow0 + d);
      bv1[tt] = *reinterpret_cast<const float4*>(krow1 + d);
    }
#pragma unroll
    for (int tt = 0; tt < TH; ++tt) {
      const float4 z = make_float4(0.f, 0.f, 0.f, 0.f);
      const float4 a = qin ? av[tt] : z;
      const float4 b0 = kin0 ? bv0[tt] : z;
      const float4 b1 = kin1 ? bv1[tt] : z;
      acc0 = __builtin_amdgcn_mfma_f32_32x32x2f32(a.x, b0.x, acc0, 0, 0, 0);
      acc1 = __builtin_amdgcn_mfma_f32_32x32x2f32(a.x, b1.x, acc1, 0, 0, 0);
      acc0 = __builtin_amdgcn_mfma_f32_32x32x2f32(a.y, b0.y, acc0, 0, 0, 0);
      acc1 = __builtin_amdgcn_mfma_f32_32x32x2f32(a.y, b1.y, acc1, 0, 0, 0);
      acc0 = __builtin_amdgcn_mfma_f32_32x32x2f32(a.z, b0.z, acc0, 0, 0, 0);
      acc1 = __builtin_amdgcn_mfma_f32_32x32x2f32(a.z, b1.z, acc1, 0, 0, 0);
      acc0 = __builtin_amdgcn_mfma_f32_32x32x2f32(a.w, b0.w, acc0, 0, 0, 0);
      acc1 = __builtin_amdgcn_mfma_f32_32x32x2f32(a.w, b1.w, acc1, 0, 0, 0);
    }
  }
  // acc0[r] / acc1[r]: row i0 + 8 (r/4) + 4 h + r%4, column j0 + m / j0 + 32 + m.
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int i = i0 + 8 * (r >> 2) + 4 * h + (r & 3);
    if (i < nc) {
      float* srow = scores + (bh * nc + i) * nc;
      if (kin0) srow[j0 + m] = acc0[r];
      if (kin1) srow[j0 + 32 + m] = acc1[r];
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

// One wavefront per score row; MAXV keys per lane (nc <= 64 * MAXV).  The
// k-th largest key is found bit by bit from the top: the largest threshold t
// with count(key >= t) >= k.  The upper 16 bits are searched over all keys.
// The k-th key then lies in the bucket of keys that share those 16 bits; the
// keys above the bucket number fewer than k.  When the bucket holds at most
// 64 keys (the usual case: about k / 2^16 of the row's spread), they are
// compacted to one per lane through LDS and the lower 16 bits are searched
// over them alone (one ballot per step instead of MAXV); otherwise (many equal
// or nearly equal scores) over all keys as before.  Either way the threshold
// is the same exact k-th largest key.
template <int MAXV>
__global__ void __launch_bounds__(256) topk_rows(const float* __restrict__ scores, int32_t* __restrict__ idx,
                                                 long long nrows, int nc, int k) {
  __shared__ uint32_t bucket[4][64];  // per wavefront
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const long long row = (long long)blockIdx.x * 4 + wv;
  if (row >= nrows) return;  // whole wavefront leaves together (no workgroup barrier below)
  const float* sr = scores + row * nc;
  uint32_t key[MAXV];
#pragma unroll
  for (int v = 0; v < MAXV; ++v) {
    const int j = v * 64 + lane;
    key[v] = (j < nc) ? order_key(sr[j]) : 0u;
  }
  const auto in = [&](int v) { return v * 64 + lane < nc; };
  uint32_t thr = 0;
  for (int bit = 31; bit >= 16; --bit) {
    const uint32_t cand = thr | (1u << bit);
    int cnt = 0;
#pragma unroll
    for (int v = 0; v < MAXV; ++v) cnt += ballot_count(in(v) && key[v] >= cand);
    if (cnt >= k) thr = cand;
  }
  const uint32_t hi = thr >> 16;
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  int above = 0, nb = 0;
#pragma unroll
  for (int v = 0; v < MAXV; ++v) {
    above += ballot_count(in(v) && (key[v] >> 16) > hi);
    const bool inb = in(v) && (key[v] >> 16) == hi;
    const uint64_t m = __ballot(inb);
    const int pos = nb + __popcll(m & lt_mask);
    if (inb && pos < 64) bucket[wv][pos] = key[v];
    nb += __popcll(m);
  }
  int gt;
  if (nb <= 64) {
    // The wavefront's own LDS writes above, read back by other lanes: LDS
    // operations of one wavefront complete in order; the fences keep the
    // compiler from moving the reads above the writes.
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const bool has = lane < nb;
    const uint32_t c = has ? bucket[wv][lane] : 0u;
    for (int bit = 15; bit >= 0; --bit) {
      const uint32_t cand = thr | (1u << bit);
      if (above + ballot_count(has && c >= cand) >= k) thr = cand;
    }
    gt = above + ballot_count(has && c > thr);
  } else {
    for (int bit = 15; bit >= 0; --bit) {
      const uint32_t cand = thr | (1u << bit);
      int cnt = 0;
#pragma unroll
      for (int v = 0; v < MAXV; ++v) cnt += ballot_count(in(v) && key[v] >= cand);
      if (cnt >= k) thr = cand;
    }
    gt = 0;
#pragma unroll
    for (int v = 0; v < MAXV; ++v) gt += ballot_count(in(v) && key[v] > thr);
  }
  const int need_eq = k - gt;  // >= 1
  int base = 0, eq_seen = 0;
  int32_t* out = idx + row * k;
#pragma unroll
  for (int v = 0; v < MAXV; ++v) {
    const int j = v * 64 + lane;
    const bool is_gt = in(v) && key[v] > thr;
    const bool is_eq = in(v) && key[v] == thr;
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
  const int ti = (g.nc + 31) / 32, tj = (g.nc + 63) / 64;
  const long long units = (long long)bh * ti * tj, per_xcd = (units + 7) / 8;
  const dim3 grid((unsigned)(8 * per_xcd));
  if (g.D == 64)
    hipLaunchKernelGGL(block_score<64>, grid, dim3(64), 0, s, qbar, kbar, scores, g.nc, ti, tj, per_xcd, units);
  else
    hipLaunchKernelGGL(block_score<128>, grid, dim3(64), 0, s, qbar, kbar, scores, g.nc, ti, tj, per_xcd, units);
  const long long nrows = (long long)bh * g.nc;
  const int per_lane = (g.nc + 63) / 64;
  // Every keys-per-lane count up to 8 has its own instantiation, larger ones
  // come in steps of a quarter to a half (each step of the search over all
  // keys costs one ballot per key slot).
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
