// Backward of the fine stage: dQ, dK, dV of block-sparse attention over the
// selected 64x64 cube blocks, from the forward's log-sum-exp.
//
// VSA is trained inside the sparse distillation (FastVideo sparse-distillation
// article, sections "核心技术解析" and "2. 视频稀疏注意力VSA"), and SLA is a
// trainable sparse-linear attention (TurboDiffusion article, section
// "稀疏、蒸馏与全链路量化"), so the block-sparse attention needs its gradient.
// For a loss with output gradient dO, per query cube i and each selected key
// cube j (the chain rule through the masked block softmax):
//   P_ij = exp(scale Q_i K_j^T - lse_i),   delta_i = rowsum(dO_i * O_i),
//   dV_j += P_ij^T dO_i,   dP_ij = dO_i V_j^T,   dS_ij = P_ij * (dP_ij - delta_i),
//   dQ_i += scale dS_ij K_j,   dK_j += scale dS_ij^T Q_i.
//
// Kernels.  No atomics: every sum is owned by one workgroup, so the results
// do not depend on scheduling.
//  * bwd_delta: delta per row (and lse in log2 units).
//  * bwd_count / bwd_scan / bwd_fill: the block lists transposed, i.e. for
//    every key cube the ascending list of query cubes whose (ascending) list
//    holds it, found by binary search.
//  * bwd_dq: one workgroup per query cube, S^T = K Q^T as in the forward (a
//    lane owns a query column); per selected block it streams K_j and V_j
//    (token-major) and K_j^T (the cube stored transposed), and accumulates
//    dQ^T = K^T dS^T.
//  * bwd_dkdv: one workgroup per key cube, S = Q K^T (a lane owns a key
//    column; Q rows in pi order, so the accumulator is the B operand of the
//    next product); K_j, V_j stay in registers; per query cube that selected
//    j it streams Q_i, dO_i (token-major), Q_i^T, dO_i^T, lse_i and delta_i,
//    and accumulates dV^T = dO^T P and dK^T = Q^T dS.
// Both stream tiles into LDS by direct buffer->LDS loads (bwd_dq one block
// ahead, bwd_dkdv two cubes ahead) and split each block by 32-row halves as
// the forward does, merging the halves through LDS.
#include <math.h>

#include "tile_pipeline.h"

namespace vsa {

namespace {

using namespace tiles;
constexpr float kLog2e = 1.4426950408889634f;

// ---------------------------------------------------------------- delta --

// delta per row, and the forward's lse in log2 units (lse log2 e) for bwd_dkdv.
template <int D>
__global__ void __launch_bounds__(256) bwd_delta(const uint16_t* __restrict__ o, const uint16_t* __restrict__ dout,
                                                 const float* __restrict__ lse, float* __restrict__ delta,
                                                 float* __restrict__ lse2, long long rows) {
  constexpr int TPR = D / 8;  // threads per row, one 16-byte chunk each
  const long long t = blockIdx.x * 256LL + threadIdx.x;
  const long long row = t / TPR;
  const int c = (int)(t % TPR);
  float sum = 0.f;
  if (row < rows) {
    const uint4 a = reinterpret_cast<const uint4*>(o + row * D)[c];
    const uint4 d = reinterpret_cast<const uint4*>(dout + row * D)[c];
    const uint32_t wa[4] = {a.x, a.y, a.z, a.w}, wd[4] = {d.x, d.y, d.z, d.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      sum = fmaf(__uint_as_float(wa[e] << 16), __uint_as_float(wd[e] << 16), sum);
      sum = fmaf(__uint_as_float(wa[e] & 0xFFFF0000u), __uint_as_float(wd[e] & 0xFFFF0000u), sum);
    }
  }
#pragma unroll
  for (int off = TPR / 2; off > 0; off >>= 1) sum += __shfl_xor(sum, off);
  if (c == 0 && row < rows) {
    delta[row] = sum;
    lse2[row] = lse[row] * kLog2e;
  }
}

// ------------------------------------------------- transposed block lists --

// Does the ascending list row[0..k) hold j?
__device__ __forceinline__ bool row_has(const int32_t* __restrict__ row, int k, int j) {
  int lo = 0, hi = k;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (row[mid] < j) lo = mid + 1;
    else hi = mid;
  }
  return lo < k && row[lo] == j;
}

// One wavefront per (b, h, key cube j): how many query cubes selected j.
__global__ void __launch_bounds__(256) bwd_count(const int32_t* __restrict__ idx, int topk, int32_t* __restrict__ cnt,
                                                 KGeom g) {
  const int lane = threadIdx.x & 63;
  const int j = blockIdx.x * 4 + (threadIdx.x >> 6);
  const long long bh = blockIdx.y;
  if (j >= g.nc) return;  // no barrier in this kernel
  const int32_t* rows = idx + bh * g.nc * (long long)topk;
  int c = 0;
  for (int i0 = 0; i0 < g.nc; i0 += 64) {
    const int i = i0 + lane;
    const bool has = i < g.nc && row_has(rows + (long long)i * topk, topk, j);
    c += __popcll(__builtin_amdgcn_ballot_w64(has));
  }
  if (lane == 0) cnt[bh * g.nc + j] = c;
}

// Exclusive prefix sum of the counts over the key cubes of one (b, h).
__global__ void __launch_bounds__(256) bwd_scan(const int32_t* __restrict__ cnt, int32_t* __restrict__ off, KGeom g) {
  __shared__ int32_t part[256];
  const long long base = (long long)blockIdx.x * g.nc;
  const int per = (g.nc + 255) / 256;
  const int lo = min((int)threadIdx.x * per, g.nc), hi = min(lo + per, g.nc);
  int s = 0;
  for (int j = lo; j < hi; ++j) s += cnt[base + j];
  part[threadIdx.x] = s;
  __syncthreads();
  for (int d = 1; d < 256; d <<= 1) {
    const int v = (int)threadIdx.x >= d ? part[threadIdx.x - d] : 0;
    __syncthreads();
    part[threadIdx.x] += v;
    __syncthreads();
  }
  int run = part[threadIdx.x] - s;
  for (int j = lo; j < hi; ++j) {
    off[base + j] = run;
    run += cnt[base + j];
  }
}

// Same search as bwd_count; the query cubes are written in ascending order.
__global__ void __launch_bounds__(256) bwd_fill(const int32_t* __restrict__ idx, int topk,
                                                const int32_t* __restrict__ off, int32_t* __restrict__ qlist,
                                                KGeom g) {
  const int lane = threadIdx.x & 63;
  const int j = blockIdx.x * 4 + (threadIdx.x >> 6);
  const long long bh = blockIdx.y;
  if (j >= g.nc) return;
  const int32_t* rows = idx + bh * g.nc * (long long)topk;
  int32_t* dst = qlist + bh * g.nc * (long long)topk + off[bh * g.nc + j];
  int run = 0;
  for (int i0 = 0; i0 < g.nc; i0 += 64) {
    const int i = i0 + lane;
    const bool has = i < g.nc && row_has(rows + (long long)i * topk, topk, j);
    const uint64_t m = __builtin_amdgcn_ballot_w64(has);
    if (has) {
      const int pos = __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0));
      dst[run + pos] = i;
    }
    run += __popcll(m);
  }
}

// 64 consecutive floats (one cube's rows of lse or delta) into LDS: one
// dword per lane of the calling wavefront.
__device__ __forceinline__ void issue_row_f32(const float* src, float* dst, int lane) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(make_rsrc(src, 256), (lds_ptr_t)dst, 4, lane * 4, 0, 0, 0);
}

// --------------------------------------------------------------------- dQ --

template <int D>
struct DqSmem {
  uint16_t k[2][64 * D];  // K_j token-major (kt_swz: also read transposed)
  uint16_t v[2][64 * D];  // V_j token-major
};

template <int D>
__device__ __forceinline__ void dq_issue(const uint16_t* kc, const uint16_t* vc, long long off, uint16_t* ks,
                                         uint16_t* vs, int w, const uint32_t* kto, const uint32_t* ko) {
  issue_k_tile<D>(make_rsrc(kc + off, 64 * D * 2), ks, w, kto);
  issue_k_tile<D>(make_rsrc(vc + off, 64 * D * 2), vs, w, ko);
}

template <int D, bool PARTIAL>
__global__ void __launch_bounds__(kThreads, 2) bwd_dq(const uint16_t* __restrict__ qc, const uint16_t* __restrict__ kc,
                                                      const uint16_t* __restrict__ vc,
                                                      const uint16_t* __restrict__ doc,
                                                      const float* __restrict__ lse, const float* __restrict__ delta,
                                                      const int32_t* __restrict__ idx, int topk, float scale,
                                                      float scale_log2, uint16_t* __restrict__ dq, KGeom g,
                                                      Placement pl) {
  constexpr int DC = D / 16, DT = D / 32;
  __shared__ __attribute__((aligned(16))) DqSmem<D> sm;
  int i, h, b;
  if (!map_workgroup(g, pl, i, h, b)) return;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wq = w & 1, wk = w >> 1;
  const int hf = lane >> 5, n = lane & 31;
  const long long bh = (long long)b * g.H + h;
  const long long hbase = bh * g.Np * D;
  const int32_t* irow = idx + (bh * g.nc + i) * topk;
  const long long row = bh * g.Np + 64LL * i + 32 * wq + n;
  const TileOffsets<D> toff(w, lane);
  const TileOffsets<D, true> ttoff(w, lane);

  dq_issue<D>(kc + hbase, vc + hbase, 64LL * irow[0] * D, sm.k[0], sm.v[0], w, ttoff.k, toff.k);
  bf16x8 qf[DC], df[DC];
#pragma unroll
  for (int dc = 0; dc < DC; ++dc) {
    qf[dc] = *reinterpret_cast<const bf16x8*>(qc + row * D + 16 * dc + 8 * hf);
    df[dc] = *reinterpret_cast<const bf16x8*>(doc + row * D + 16 * dc + 8 * hf);
  }
  const float lse2 = lse[row] * kLog2e, dl = delta[row];
  const int prow = pi_row(n);
  f32x16 acc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) acc[dt] = f32x16{};

  for (int jb = 0; jb < topk; jb += 2) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int nb = jb + u;
      if (nb < topk) {
        wait_vmcnt<0>();
        pipeline_barrier();
        if (nb + 1 < topk)
          dq_issue<D>(kc + hbase, vc + hbase, 64LL * irow[nb + 1] * D, sm.k[u ^ 1], sm.v[u ^ 1], w, ttoff.k,
                      toff.k);
        bf16x8 ka[DC], va[DC];
        read_k<D, true>(sm.k[u], wk, hf, prow, ka);
        read_k<D>(sm.v[u], wk, hf, prow, va);
        f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
        for (int dc = 0; dc < DC; ++dc) {
          s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[dc], qf[dc], s, 0, 0, 0);
          dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[dc], df[dc], dp, 0, 0, 0);
        }
        if (PARTIAL) mask_keys(s, g, irow[nb], wk, hf);
        uint32_t sw[8];
#pragma unroll
        for (int r = 0; r < 8; ++r) {
          const float p0 = __builtin_amdgcn_exp2f(fmaf(s[2 * r], scale_log2, -lse2));
          const float p1 = __builtin_amdgcn_exp2f(fmaf(s[2 * r + 1], scale_log2, -lse2));
          const f32x2 d2 = {p0 * (dp[2 * r] - dl), p1 * (dp[2 * r + 1] - dl)};
          sw[r] = __builtin_bit_cast(uint32_t, __builtin_convertvector(d2, bf16x2));
        }
        const bf16x8 sb[2] = {__builtin_bit_cast(bf16x8, make_uint4(sw[0], sw[1], sw[2], sw[3])),
                              __builtin_bit_cast(bf16x8, make_uint4(sw[4], sw[5], sw[6], sw[7]))};
        bf16x8 ta[DT][2];
        read_tr<D>(sm.k[u], wk, lane, ta);
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
          for (int kk = 0; kk < 2; ++kk) acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ta[dt][kk], sb[kk], acc[dt], 0, 0, 0);
      }
    }
  }

  // The two key halves hold partial sums of the same dQ^T: add them.
  wait_vmcnt<0>();
  __syncthreads();
  float* xo = reinterpret_cast<float*>(&sm) + wq * (DT * 16 * 64);
  if (wk == 1) {
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) xo[(dt * 16 + r) * 64 + lane] = acc[dt][r];
  }
  __syncthreads();
  if (wk == 1) return;
  uint16_t* orow = dq + row * D;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int gq = 0; gq < 4; ++gq) {
      float v[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 4 * gq + e;
        v[e] = scale * (acc[dt][r] + xo[(dt * 16 + r) * 64 + lane]);
      }
      *reinterpret_cast<uint2*>(orow + 32 * dt + 8 * gq + 4 * hf) =
          make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
    }
}

// ------------------------------------------------------------------ dK dV --
//
// One workgroup of 8 wavefronts per key cube j.  Wavefronts 0-3 and 4-7
// split the work of each (key, query) quadrant (wk, wq), 32 keys x 32 queries,
// by product, so that each SIMD holds one of each kind:
//  * P wavefronts (0-3): S = Q K^T, P = exp(scale S - lse), dV^T += dO^T P;
//    they hand P (fp32) to their partner through LDS;
//  * dS wavefronts (4-7), one cube behind: dP = dO V^T, dS = P * (dP - delta),
//    dK^T += Q^T dS.
// Every step has two phases split by a barrier.  In phase A the P wavefronts
// read their operands for cube m from LDS while the dS wavefronts run their
// products for cube m - 1 on operands already in registers; in phase B the
// roles swap: the P wavefronts run cube m, the dS wavefronts read cube m.  So
// on every SIMD one wavefront reads while the other computes, and the LDS
// reads of the step no longer all land at once after a single barrier.
// A lane owns a key column (S = Q K^T with Q rows in pi order, so the
// accumulator is the B operand of the next product); K (P wavefronts) or V
// (dS wavefronts) stays in registers.
//
// Tiles: P wavefronts load Q and lse, dS wavefronts dO and delta, each two
// cubes ahead into a ring of three, right after their own reads of the step.
// A wavefront waits for its previous loads just before those reads (one step
// after issuing them); every reader of that cube comes at least one barrier
// later.  The ring slot a load overwrites was last read in the previous step.
// That wait also leaves no tile load of the wavefront in flight when it issues
// ds_read_b64_tr_b16, for which the compiler waits for all of them.

template <int N>
struct SlotC {
  static constexpr int value = N;
};

template <int D>
struct DkvSmem {
  uint16_t q[3][64 * D];     // Q_i token-major (kt_swz: also read transposed)
  uint16_t dout[3][64 * D];  // dO_i token-major (kt_swz)
  float ls[3][64];           // lse_i log2 e
  float dl[3][64];           // delta_i
  f32x4 p[4][4][64];         // P of one cube: [quadrant][register / 4][lane]
};

template <int D, bool PARTIAL>
__global__ void __launch_bounds__(2 * kThreads, 1) bwd_dkdv(const uint16_t* __restrict__ qc,
                                                            const uint16_t* __restrict__ kc,
                                                            const uint16_t* __restrict__ vc,
                                                            const uint16_t* __restrict__ doc,
                                                            const float* __restrict__ lse2,
                                                            const float* __restrict__ delta,
                                                            const int32_t* __restrict__ qoff,
                                                            const int32_t* __restrict__ qcnt,
                                                            const int32_t* __restrict__ qlist, int topk, float scale,
                                                            float scale_log2, uint16_t* __restrict__ dk,
                                                            uint16_t* __restrict__ dv, KGeom g, Placement pl) {
  constexpr int DC = D / 16, DT = D / 32;
  __shared__ __attribute__((aligned(16))) DkvSmem<D> sm;
  int j, h, b;
  if (!map_workgroup(g, pl, j, h, b)) return;  // whole workgroup leaves before any barrier
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool ds_wave = w >= 4;  // false: P wavefront
  const int quad = w & 3, wk = quad & 1, wq = quad >> 1;
  const int hf = lane >> 5, n = lane & 31;
  const int key = 32 * wk + n;
  const long long bh = (long long)b * g.H + h;
  const long long hbase = bh * g.Np * D, rbase = bh * g.Np;
  const long long krow = rbase + 64LL * j + key;
  const TileOffsets<D, true> toff(quad, lane);
  const int cnt = qcnt[bh * g.nc + j];
  const int32_t* list = qlist + bh * (long long)g.nc * topk + qoff[bh * g.nc + j];
  // P wavefronts load the Q tiles and lse log2 e, dS wavefronts the dO tiles and delta.
  const uint16_t* src = (ds_wave ? doc : qc) + hbase;
  const float* rsrc_f = ds_wave ? delta : lse2;
  auto issue = [&](int m, int slot) {
    const int i = list[m];
    issue_k_tile<D>(make_rsrc(src + 64LL * i * D, 64 * D * 2), ds_wave ? sm.dout[slot] : sm.q[slot], quad, toff.k);
    if (quad == 0) issue_row_f32(rsrc_f + rbase + 64LL * i, ds_wave ? sm.dl[slot] : sm.ls[slot], lane);
  };
  if (cnt > 0) issue(0, 0);
  if (cnt > 1) issue(1, 1);

  // This wavefront's 32 keys of K (P) or V (dS), B operand fragments.
  bf16x8 kv[DC];
  {
    const uint16_t* kvrow = (ds_wave ? vc : kc) + krow * D;
#pragma unroll
    for (int dc = 0; dc < DC; ++dc) kv[dc] = *reinterpret_cast<const bf16x8*>(kvrow + 16 * dc + 8 * hf);
  }
  float kmask = 1.f;
  if (PARTIAL) {
    int ct, cy, cx;
    cube_coords(g, j, ct, cy, cx);
    kmask = local_valid(g, ct, cy, cx, key) ? 1.f : 0.f;
  }
  const int prow = pi_row(n);
  // Register r of a 32 x 32 accumulator holds query 32 wq + 16 (r/8) + 8 hf + r%8.
  const int q0 = 32 * wq + 8 * hf;
  f32x16 acc[DT];  // dV^T (P wavefronts) or dK^T (dS wavefronts)
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) acc[dt] = f32x16{};
  // The transposed operand is read one phase ahead of its product: dO^T (P)
  // or Q^T (dS).  The row operands are read right before their products.
  bf16x8 ta[DT][2];
  bf16x8 bop[2];  // B operand of the deferred product: P (P wavefronts) or dS (dS wavefronts), bf16
  f32x4* const pslot = &sm.p[quad][0][lane];
  wait_vmcnt<0>();  // the first two cubes

  // Ring slots: cube m in m % 3, unrolled by three so that every slot base is
  // a compile-time constant in the instruction offset.  Each read kind adds
  // it to a loop-invariant lane offset that already holds its ring's base, so
  // no offset exceeds the 64 KB an instruction reaches and the loops compute
  // no LDS address.  The two kinds run separate loops with the same barriers:
  // two per step, steps m = 0 .. cnt.
  constexpr uint32_t kTile = 64 * D * 2;  // bytes per Q or dO tile
  const char* const lds0 = reinterpret_cast<const char*>(&sm);
  const uint32_t q_base = (uint32_t)(reinterpret_cast<const char*>(&sm.q[0][0]) - lds0);
  const uint32_t d_base = (uint32_t)(reinterpret_cast<const char*>(&sm.dout[0][0]) - lds0);
  // Row operand (A of S or dP; rows 32 wq + pi order) and transposed operand
  // (A of dV^T or dK^T, read_tr_one's lane layout, kk = 0) of this wavefront,
  // byte offsets within a tile, plus the base of the ring each kind reads.
  uint32_t ko[DC], to[2 * DT];
  {
    const int krow = 32 * wq + prow;
    const uint32_t rb = ds_wave ? d_base : q_base;
#pragma unroll
    for (int dc = 0; dc < DC; ++dc)
      ko[dc] = rb + (uint32_t)(krow * D + (((2 * dc + hf) ^ kt_swz<D>(krow)) * 8)) * 2u;
    const int s = lane & 15, grp = lane >> 4;
    const uint32_t tb = ds_wave ? q_base : d_base;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int r = 32 * wq + 8 * hf + 4 * h + (s >> 2);
        const int d = 32 * dt + 16 * (grp & 1) + 4 * (s & 3);
        to[2 * dt + h] = tb + (uint32_t)(r * D + (((d >> 3) ^ kt_swz<D>(r)) << 3) + (d & 4)) * 2u;
      }
    // Opaque to the optimiser, so that it keeps these sums and puts only the
    // slot's constant into each instruction.
#pragma unroll
    for (int dc = 0; dc < DC; ++dc) asm volatile("" : "+v"(ko[dc]));
#pragma unroll
    for (int e = 0; e < 2 * DT; ++e) asm volatile("" : "+v"(to[e]));
  }
  auto read_rows = [&](uint32_t slot_off, bf16x8(&xa)[DC]) {
#pragma unroll
    for (int dc = 0; dc < DC; ++dc) xa[dc] = *reinterpret_cast<const bf16x8*>(lds0 + ko[dc] + slot_off);
  };
  auto read_cols = [&](uint32_t slot_off) {
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        i16x4 part[2];
#pragma unroll
        for (int h = 0; h < 2; ++h)
          part[h] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (lds_i16x4_ptr)(lds0 + to[2 * dt + h] + slot_off + kk * 16 * D * 2));
        ta[dt][kk] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(part[0], part[1], 0, 1, 2, 3, 4, 5, 6, 7));
      }
  };
  auto dmma = [&]() {  // the deferred product: acc += ta bop
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
        acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ta[dt][kk], bop[kk], acc[dt], 0, 0, 0);
  };
  const int steps = cnt > 0 ? cnt + 1 : 0;
  if (!ds_wave) {
    auto step = [&](int m, auto slot) {
      constexpr int S = decltype(slot)::value, S2 = (S + 2) % 3;
      pipeline_barrier();
      // Phase A: dV^T += dO(m-1)^T P(m-1) on registers, then dO(m)^T into
      // registers and the loads of Q(m + 2).
      if (m >= 1) dmma();
      if (m < cnt) {
        wait_vmcnt<0>();  // Q(m + 1), read from the next step on
        read_cols(S * kTile);
        if (m + 2 < cnt) issue(m + 2, S2);
      }
      pipeline_barrier();
      // Phase B: S = Q(m) K^T, P = exp(scale S - lse) to LDS and, as bf16,
      // to the next phase A.
      if (m < cnt) {
        bf16x8 xa[DC];
        read_rows(S * kTile, xa);
        __builtin_amdgcn_sched_barrier(0);  // all row reads in flight before the chain
        f32x16 x = f32x16{};
#pragma unroll
        for (int dc = 0; dc < DC; ++dc) x = __builtin_amdgcn_mfma_f32_32x32x16_bf16(xa[dc], kv[dc], x, 0, 0, 0);
        const f32x4* lsp = reinterpret_cast<const f32x4*>(&sm.ls[S][0]);
        const f32x4 l4[4] = {lsp[q0 / 4], lsp[q0 / 4 + 1], lsp[(q0 + 16) / 4], lsp[(q0 + 16) / 4 + 1]};
        f32x4 pv[4];
#pragma unroll
        for (int r = 0; r < 16; ++r)
          pv[r / 4][r % 4] = kmask * __builtin_amdgcn_exp2f(fmaf(x[r], scale_log2, -l4[r / 4][r % 4]));
#pragma unroll
        for (int c = 0; c < 4; ++c) pslot[64 * c] = pv[c];
        uint32_t bw[8];
#pragma unroll
        for (int r = 0; r < 8; ++r) {
          const f32x2 p2 = {pv[r / 2][2 * (r % 2)], pv[r / 2][2 * (r % 2) + 1]};
          bw[r] = __builtin_bit_cast(uint32_t, __builtin_convertvector(p2, bf16x2));
        }
        bop[0] = __builtin_bit_cast(bf16x8, make_uint4(bw[0], bw[1], bw[2], bw[3]));
        bop[1] = __builtin_bit_cast(bf16x8, make_uint4(bw[4], bw[5], bw[6], bw[7]));
      }
    };
    int m = 0;
    for (; m + 3 <= steps; m += 3) {  // full groups: no per-step guard, no register copies between steps
      step(m, SlotC<0>{});
      step(m + 1, SlotC<1>{});
      step(m + 2, SlotC<2>{});
    }
    if (m < steps) step(m, SlotC<0>{});
    if (m + 1 < steps) step(m + 1, SlotC<1>{});
  } else {
    auto step = [&](int m, auto slot) {
      constexpr int S = decltype(slot)::value, S2 = (S + 2) % 3;  // S2: also (m - 1) % 3
      pipeline_barrier();
      // Phase A, cube m - 1: dP = dO V^T, dS = P * (dP - delta) in bf16 for
      // the next phase B.
      if (m >= 1) {
        bf16x8 xa[DC];
        read_rows(S2 * kTile, xa);
        __builtin_amdgcn_sched_barrier(0);  // all row reads in flight before the chain
        f32x16 x = f32x16{};
#pragma unroll
        for (int dc = 0; dc < DC; ++dc) x = __builtin_amdgcn_mfma_f32_32x32x16_bf16(xa[dc], kv[dc], x, 0, 0, 0);
        const f32x4* dlp = reinterpret_cast<const f32x4*>(&sm.dl[S2][0]);
        const f32x4 d4[4] = {dlp[q0 / 4], dlp[q0 / 4 + 1], dlp[(q0 + 16) / 4], dlp[(q0 + 16) / 4 + 1]};
        f32x4 pv[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) pv[c] = pslot[64 * c];
        uint32_t bw[8];
#pragma unroll
        for (int r = 0; r < 8; ++r) {
          const int r0 = 2 * r, r1 = 2 * r + 1;
          const f32x2 d2 = {pv[r0 / 4][r0 % 4] * (x[r0] - d4[r0 / 4][r0 % 4]),
                            pv[r1 / 4][r1 % 4] * (x[r1] - d4[r1 / 4][r1 % 4])};
          bw[r] = __builtin_bit_cast(uint32_t, __builtin_convertvector(d2, bf16x2));
        }
        bop[0] = __builtin_bit_cast(bf16x8, make_uint4(bw[0], bw[1], bw[2], bw[3]));
        bop[1] = __builtin_bit_cast(bf16x8, make_uint4(bw[4], bw[5], bw[6], bw[7]));
      }
      pipeline_barrier();
      // Phase B: dK^T += Q(m-1)^T dS on registers, then Q(m)^T into
      // registers and the loads of dO(m + 2).
      if (m >= 1) dmma();
      if (m < cnt) {
        wait_vmcnt<0>();  // dO(m + 1), read from the next step on
        read_cols(S * kTile);
        if (m + 2 < cnt) issue(m + 2, S2);
      }
    };
    int m = 0;
    for (; m + 3 <= steps; m += 3) {  // full groups: no per-step guard, no register copies between steps
      step(m, SlotC<0>{});
      step(m + 1, SlotC<1>{});
      step(m + 2, SlotC<2>{});
    }
    if (m < steps) step(m, SlotC<0>{});
    if (m + 1 < steps) step(m + 1, SlotC<1>{});
  }

  // The two query halves hold partial sums of the same dK^T (dV^T): add them.
  wait_vmcnt<0>();
  __syncthreads();
  float* x = reinterpret_cast<float*>(&sm) + ((ds_wave ? 2 : 0) + wk) * (DT * 16 * 64);
  if (wq == 1) {
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) x[(dt * 16 + r) * 64 + lane] = acc[dt][r];
  }
  __syncthreads();
  if (wq == 1) return;
  const float f = ds_wave ? scale : 1.f;
  uint16_t* out = (ds_wave ? dk : dv) + krow * D;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int gq = 0; gq < 4; ++gq) {
      float o[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 4 * gq + e;
        o[e] = f * (acc[dt][r] + x[(dt * 16 + r) * 64 + lane]);
      }
      *reinterpret_cast<uint2*>(out + 32 * dt + 8 * gq + 4 * hf) =
          make_uint2(pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]));
    }
}

// Workspace carve-up: delta [B H Np] f32 | lse log2 e [B H Np] f32 | cnt [B H Nc] | off [B H Nc] |
// list [B H Nc topk] int32.
struct BwdWs {
  float *delta, *lse2;
  int32_t *cnt, *off, *list;
};

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

inline BwdWs carve(const KGeom& g, int topk, void* ws) {
  uintptr_t p = reinterpret_cast<uintptr_t>(ws);
  const size_t bh = (size_t)g.B * g.H;
  BwdWs w;
  w.delta = reinterpret_cast<float*>(p);
  p += align256(bh * g.Np * sizeof(float));
  w.lse2 = reinterpret_cast<float*>(p);
  p += align256(bh * g.Np * sizeof(float));
  w.cnt = reinterpret_cast<int32_t*>(p);
  p += align256(bh * g.nc * sizeof(int32_t));
  w.off = reinterpret_cast<int32_t*>(p);
  p += align256(bh * g.nc * sizeof(int32_t));
  w.list = reinterpret_cast<int32_t*>(p);
  return w;
}

template <int D, bool PARTIAL>
hipError_t launch_bwd_t(const KGeom& g, const uint16_t* qc, const uint16_t* kc, const uint16_t* vc,
                        const uint16_t* oc, const uint16_t* doc, const float* lse, const int32_t* idx, int topk,
                        float scale, uint16_t* dq, uint16_t* dk, uint16_t* dv, void* ws, hipStream_t s) {
  const BwdWs w = carve(g, topk, ws);
  const long long rows = (long long)g.B * g.H * g.Np;
  bwd_delta<D><<<dim3((unsigned)((rows * (D / 8) + 255) / 256)), dim3(256), 0, s>>>(oc, doc, lse, w.delta, w.lse2,
                                                                                    rows);
  const dim3 tgrid((g.nc + 3) / 4, g.B * g.H);
  bwd_count<<<tgrid, dim3(256), 0, s>>>(idx, topk, w.cnt, g);
  bwd_scan<<<dim3(g.B * g.H), dim3(256), 0, s>>>(w.cnt, w.off, g);
  bwd_fill<<<tgrid, dim3(256), 0, s>>>(idx, topk, w.off, w.list, g);
  const Placement pl = make_placement(g);
  const float scale_log2 = scale * kLog2e;
  bwd_dq<D, PARTIAL><<<dim3(grid_size(g)), dim3(kThreads), 0, s>>>(qc, kc, vc, doc, lse, w.delta, idx, topk, scale,
                                                                    scale_log2, dq, g, pl);
  bwd_dkdv<D, PARTIAL><<<dim3(grid_size(g)), dim3(2 * kThreads), 0, s>>>(qc, kc, vc, doc, w.lse2, w.delta, w.off, w.cnt,
                                                                      w.list, topk, scale, scale_log2, dk, dv, g, pl);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_block_lists_t(const KGeom& g, const int32_t* idx, int topk, int32_t* cnt, int32_t* off,
                                int32_t* list, hipStream_t s) {
  const dim3 tgrid((g.nc + 3) / 4, g.B * g.H);
  bwd_count<<<tgrid, dim3(256), 0, s>>>(idx, topk, cnt, g);
  bwd_scan<<<dim3(g.B * g.H), dim3(256), 0, s>>>(cnt, off, g);
  bwd_fill<<<tgrid, dim3(256), 0, s>>>(idx, topk, off, list, g);
  return hipGetLastError();
}

size_t attn_bwd_workspace_bytes(const KGeom& g, int topk) {
  const size_t bh = (size_t)g.B * g.H;
  return 2 * align256(bh * g.Np * sizeof(float)) + 2 * align256(bh * g.nc * sizeof(int32_t)) +
         align256(bh * g.nc * (size_t)topk * sizeof(int32_t));
}

hipError_t launch_attn_bwd(const KGeom& g, const uint16_t* qc, const uint16_t* kc, const uint16_t* vc,
                           const uint16_t* oc, const uint16_t* doc, const float* lse, const int32_t* idx, int topk,
                           float scale, uint16_t* dq, uint16_t* dk, uint16_t* dv, void* ws, hipStream_t s) {
  if (g.D == 64) {
    if (g.partial) return launch_bwd_t<64, true>(g, qc, kc, vc, oc, doc, lse, idx, topk, scale, dq, dk, dv, ws, s);
    return launch_bwd_t<64, false>(g, qc, kc, vc, oc, doc, lse, idx, topk, scale, dq, dk, dv, ws, s);
  }
  if (g.partial) return launch_bwd_t<128, true>(g, qc, kc, vc, oc, doc, lse, idx, topk, scale, dq, dk, dv, ws, s);
  return launch_bwd_t<128, false>(g, qc, kc, vc, oc, doc, lse, idx, topk, scale, dq, dk, dv, ws, s);
}

}  // namespace vsa
