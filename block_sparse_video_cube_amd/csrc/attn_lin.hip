// Fine stage fused with the linear branch: O = O_sparse + O_lin in one pass.
//
// A block-sparse branch paired with a linear branch keeps global context when
// most blocks are skipped (SparkDiffusion article, paragraph 3, RoLA;
// TurboDiffusion article, section "稀疏、蒸馏与全链路量化", SLA).  The
// linear branch over the unselected cubes U of query cube i is
//   O_lin = phi(Q) (sum_U phi(K)^T V) / (phi(Q) . sum_U phi(K)),  phi = elu + 1,
// taken as the total state minus the selected part (as linear.hip does):
//   num = phi(Q) S_tot - sum_{j in sel} (phi(Q) phi(K_j)^T) V_j
//   den = phi(Q) z_tot - sum_{j in sel} rowsum(phi(Q) phi(K_j)^T).
// The selected part needs the very K and V tiles the fine stage streams, so
// one workgroup of 8 wavefronts runs both branches on one tile pipeline:
//  * wavefronts 0-3 are the fine stage of attn_fwd.hip (same step, same
//    split: wavefront (wq, wk) owns queries 32 wq .. +31, keys 32 wk .. +31)
//    and the only ones that load tiles;
//  * wavefronts 4-7 run the linear branch one block behind.  In step n they
//    turn their quarter of the K(n+1) tile that just landed into phi(K) rows
//    in a second LDS ring (bf16, zero on padded keys: the values lin_state
//    writes to HBM for the two-call chain), and multiply with phi(K(n)) from
//    that ring and with the V(n-1) tile the softmax wavefronts read in the
//    same step: S'^T(n) = phiK(n) phiQ^T, C^T -= V(n-1)^T P'(n-1)^T.  They
//    start from phi(Q) S_tot (bf16 hi + lo halves, one per key-half
//    wavefront) and finish with the denominator;
//  * at the end both halves of both branches merge through LDS and the
//    wk = 0 attention wavefronts write bf16(O_sparse + O_lin) once.
// Per block the workgroup brings only the K and V tiles (32 KB at D = 128),
// like the fine stage alone: the linear branch adds no tile traffic, where
// the two-call chain reads phi(K) and V a second time.  The 8 wavefronts
// take 2 per SIMD, so one workgroup per compute unit, which then holds all
// of the compute unit's LDS for its rings.
#include <math.h>

#include "attn_core.h"

namespace vsa {

namespace {

using namespace tiles;
using namespace attn_core;

constexpr int kLinThreads = 512;

// Four-slot K and V rings: with one workgroup per compute unit, each tile is
// requested three steps before it is read, so the loads of one workgroup
// keep as many bytes in flight as two fine-stage workgroups do.  160 KB at
// D = 128, all of gfx950's LDS.
template <int D>
struct SmemL {
  uint16_t k[4][64 * D];
  uint16_t v[4][D * 64];
  uint16_t f[2][64 * D];  // phi(K) tiles, written by the linear wavefronts
};

// phi of eight bf16 values, rounded to bf16; zero for a padded key row.
__device__ __forceinline__ uint4 phi8(uint4 raw, bool valid) {
  const uint32_t wv[4] = {raw.x, raw.y, raw.z, raw.w};
  uint32_t o[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) o[e] = valid ? phi2_bf16(wv[e]) : 0u;
  return make_uint4(o[0], o[1], o[2], o[3]);
}

template <int D, bool PARTIAL>
__global__ void __launch_bounds__(kLinThreads, 1) attn_lin_fwd(
    const uint16_t* __restrict__ qc, const uint16_t* __restrict__ kc, const uint16_t* __restrict__ vt,
    const int32_t* __restrict__ idx, int topk, float scale, float scale_log2, const uint16_t* __restrict__ st_hi,
    const uint16_t* __restrict__ st_lo, const float* __restrict__ z_tot, uint16_t* __restrict__ oc,
    float* __restrict__ lse, KGeom g, Placement pl) {
  constexpr int DC = D / 16, DT = D / 32;
  constexpr int NI = TileOffsets<D>::NI, KRPI = TileOffsets<D>::KRPI;
  constexpr int XO = DT * 16 * 64;  // floats of one wq's handed-over accumulator
  // One LDS object: with several, the compiler's LDS-DMA tracking made some
  // tile reads wait for every load in flight.
  __shared__ __attribute__((aligned(16))) SmemL<D> sm;

  int i, h, b;
  if (!map_workgroup(g, pl, i, h, b)) return;  // whole workgroup leaves before any barrier
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int role = w >> 2, w4 = w & 3;  // role 0: softmax branch, 1: linear branch
  const int wq = w4 & 1, wk = w4 >> 1;
  const int hf = lane >> 5, n = lane & 31;
  const long long bh = (long long)b * g.H + h;
  const int32_t* irow = idx + (bh * g.nc + i) * topk;
  const int q = 32 * wq + n;
  const long long row = bh * g.Np + 64LL * i + q;
  const auto blk = [&](int m) { return irow[m < topk ? m : topk - 1]; };
  const int prow = pi_row(n);
  // Hand-over space once the rings are idle: accumulators in the K ring,
  // per-query scalars in the V ring.
  float* xo_att = reinterpret_cast<float*>(&sm.k[0][0]) + wq * XO;
  float* xo_lin = reinterpret_cast<float*>(&sm.k[0][0]) + (2 + wq) * XO;
  float* xm = reinterpret_cast<float*>(&sm.v[0][0]) + wq * 128;  // attention wk = 1: max, sum
  float* xd = reinterpret_cast<float*>(&sm.v[1][0]) + wq * 64;   // linear wk = 1: selected row sums

  if (role == 0) {
    // ---------------------------------------------------------------- softmax
    const TileOffsets<D> toff(w4, lane);
    const uint16_t* kbase = kc + bh * g.Np * D;
    const uint16_t* vbase = vt + bh * g.Np * D;
    constexpr unsigned kTile = 64 * D * 2;
    // Tile m of the list (past the end: a zero-size range, no memory traffic).
    const auto k_rsrc = [&](int m) { return make_rsrc(kbase + 64LL * blk(m) * D, m < topk ? kTile : 0u); };
    const auto v_rsrc = [&](int m) { return make_rsrc(vbase + 64LL * blk(m) * D, m < topk ? kTile : 0u); };
    {
      // V(-1) = 0 (slot 3), written before any tile load is in flight.
      uint4* z = reinterpret_cast<uint4*>(sm.v[3]);
#pragma unroll
      for (int e = tid; e < D * 64 * 2 / 16; e += kLinThreads / 2) z[e] = make_uint4(0, 0, 0, 0);
    }
    // K(m) and V(m) live in slot m % 4.  Step n reads K(n+1) and V(n-1) and
    // issues V(n+2) and K(n+4); the prologue issues what steps -3 .. -1
    // would have: K(0), then K(1), K(2), V(0), K(3), V(1).
    issue_k_tile<D>(k_rsrc(0), sm.k[0], w4, toff.k);
    bf16x8 qf[DC];
    {
      const uint16_t* qrow = qc + row * D;
#pragma unroll
      for (int dc = 0; dc < DC; ++dc) qf[dc] = *reinterpret_cast<const bf16x8*>(qrow + 16 * dc + 8 * hf);
    }
    issue_k_tile<D>(k_rsrc(1), sm.k[1], w4, toff.k);
    issue_k_tile<D>(k_rsrc(2), sm.k[2], w4, toff.k);
    issue_v_tile<D>(v_rsrc(0), sm.v[0], w4, toff.v);
    issue_k_tile<D>(k_rsrc(3), sm.k[3], w4, toff.k);
    issue_v_tile<D>(v_rsrc(1), sm.v[1], w4, toff.v);
    f32x16 o[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) o[dt] = f32x16{};
    float m_run = -INFINITY, l_run = 0.f;
    const float lazy_raw = kLazyLog2 / scale_log2;
    bf16x8 p_prev[2] = {};
    f32x16 s_cur;
    float mx_cur;
    {
      wait_vmcnt<5 * NI>();  // K(0) and the Q fragments
      pipeline_barrier();
      bf16x8 ka[DC];
      read_k<D>(sm.k[0], wk, hf, prow, ka);
      s_cur = f32x16{};
#pragma unroll
      for (int dc = 0; dc < DC; ++dc) s_cur = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[dc], qf[dc], s_cur, 0, 0, 0);
      if (PARTIAL) mask_keys(s_cur, g, blk(0), wk, hf);
      mx_cur = max16(s_cur);
    }
    bool move = __builtin_amdgcn_ballot_w64(mx_cur > m_run + lazy_raw) != 0;
    auto run_step = [&](int nb, auto uc) {
      constexpr int u = decltype(uc)::value;  // nb % 4
      // K(nb+1) and V(nb-1) were issued three steps back (or in the
      // prologue); at most the four tiles issued since stay in flight.
      wait_vmcnt<4 * NI>();
      pipeline_barrier();
      bf16x8 ka[DC];
      bf16x8 va[DT][2];
      read_k<D>(sm.k[(u + 1) % 4], wk, hf, prow, ka);
      read_v<D>(sm.v[(u + 3) % 4], wk, hf, n, va);
      float alpha = 1.f;
      const bool resc = move;
      if (resc) {
        const float row_max = fmaxf(mx_cur, __shfl_xor(mx_cur, 32));
        const bool grow = row_max > m_run + lazy_raw;
        alpha = grow ? __builtin_amdgcn_exp2f((m_run - row_max) * scale_log2) : 1.f;
        m_run = grow ? row_max : m_run;
        l_run *= alpha;
      }
      const float mc = (m_run == -INFINITY) ? 0.f : m_run * scale_log2;
      f32x16 s_next;
      float mx_next;
      bf16x8 p_cur[2];
      const int j_next = blk(nb + 1);
      step<D, PARTIAL>(ka, va, qf, s_cur, s_next, mx_next, p_prev, p_cur, o, l_run, mc, scale_log2,
                       [&](f32x16& s) { mask_keys(s, g, j_next, wk, hf); }, v_rsrc(nb + 2),
                       sm.v[(u + 2) % 4] + w4 * NI * 8 * 64, toff.v, k_rsrc(nb + 4),
                       sm.k[u] + w4 * NI * KRPI * D, toff.k);
      move = __builtin_amdgcn_ballot_w64(mx_next > m_run + lazy_raw) != 0;
      if (resc) {
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) o[dt] *= alpha;
      }
      s_cur = s_next;
      mx_cur = mx_next;
      p_prev[0] = p_cur[0];
      p_prev[1] = p_cur[1];
    };
    int jb = 0;
    for (; jb + 4 <= topk; jb += 4) {
      run_step(jb, StepC<0>{});
      run_step(jb + 1, StepC<1>{});
      run_step(jb + 2, StepC<2>{});
      run_step(jb + 3, StepC<3>{});
    }
    if (jb < topk) run_step(jb, StepC<0>{});
    if (jb + 1 < topk) run_step(jb + 1, StepC<1>{});
    if (jb + 2 < topk) run_step(jb + 2, StepC<2>{});
    {
      // V(topk-1): at most the four tiles issued after it remain (the K
      // loads among them past the end move no data).
      wait_vmcnt<4 * NI>();
      pipeline_barrier();
      bf16x8 va[DT][2];
      read_v<D>(sm.v[(topk - 1) & 3], wk, hf, n, va);
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
          o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[dt][kk], p_prev[kk], o[dt], 0, 0, 0);
    }
    l_run += __shfl_xor(l_run, 32);
    wait_vmcnt<0>();
    __syncthreads();  // every tile read is done: the rings become hand-over space
    if (wk == 1) {
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) xo_att[(dt * 16 + r) * 64 + lane] = o[dt][r];
      xm[lane] = m_run;
      xm[64 + lane] = l_run;
    }
    __syncthreads();
    __syncthreads();  // the linear wavefronts have left O_lin in xo_lin
    if (wk == 1) return;
    const float m1 = xm[lane], l1 = xm[64 + lane];
    const float m = fmaxf(m_run, m1);
    const float a0 = __builtin_amdgcn_exp2f((m_run - m) * scale_log2);
    const float a1 = __builtin_amdgcn_exp2f((m1 - m) * scale_log2);
    const float l_tot = l_run * a0 + l1 * a1;
    const float inv = 1.f / l_tot;
    const float c0 = a0 * inv, c1 = a1 * inv;
    uint16_t* orow = oc + row * D;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        const int d = 32 * dt + 8 * gq + 4 * hf;
        float v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 4 * gq + e;
          const float os = o[dt][r] * c0 + xo_att[(dt * 16 + r) * 64 + lane] * c1;
          v[e] = os + xo_lin[(dt * 16 + r) * 64 + lane];
        }
        *reinterpret_cast<uint2*>(orow + d) = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
      }
    if (lse && hf == 0) lse[row] = m * scale + logf(l_tot);
  } else {
    // ----------------------------------------------------------------- linear
    const bool empty_u = topk >= g.nc;  // every cube selected: O_lin = 0
    // phi(Q) fragments (bf16) and this lane's part of phi(Q) . z_tot, with
    // the Q row and the z_tot entries all loaded before use.
    bf16x8 fq[DC];
    float den_part = 0.f;
    {
      const uint16_t* qrow = qc + row * D;
      const float* zt = z_tot + bh * D + 8 * hf;
      uint4 raw[DC];
      float4 zv[DC][2];
#pragma unroll
      for (int dc = 0; dc < DC; ++dc) {
        raw[dc] = *reinterpret_cast<const uint4*>(qrow + 16 * dc + 8 * hf);
        zv[dc][0] = *reinterpret_cast<const float4*>(zt + 16 * dc);
        zv[dc][1] = *reinterpret_cast<const float4*>(zt + 16 * dc + 4);
      }
#pragma unroll
      for (int dc = 0; dc < DC; ++dc) {
        const uint32_t wv[4] = {raw[dc].x, raw[dc].y, raw[dc].z, raw[dc].w};
        const float zz[8] = {zv[dc][0].x, zv[dc][0].y, zv[dc][0].z, zv[dc][0].w,
                             zv[dc][1].x, zv[dc][1].y, zv[dc][1].z, zv[dc][1].w};
#pragma unroll
        for (int e2 = 0; e2 < 4; ++e2) {
          const uint32_t pp = phi2_bf16(wv[e2]);
          const uint16_t p0 = (uint16_t)pp, p1 = (uint16_t)(pp >> 16);
          fq[dc][2 * e2] = __builtin_bit_cast(__bf16, p0);
          fq[dc][2 * e2 + 1] = __builtin_bit_cast(__bf16, p1);
          den_part += bf16_to_f32(p0) * zz[2 * e2] + bf16_to_f32(p1) * zz[2 * e2 + 1];
        }
      }
      asm volatile("" ::"v"(den_part));  // keep the sum here, not after the loop
    }
    __builtin_amdgcn_sched_barrier(0);
    // c starts as this key half's share of phi(Q) S_tot (the hi or the lo
    // half); the steps subtract the selected part with negated weights.
    f32x16 c[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) c[dt] = f32x16{};
    mat_rows_mfma<D>((wk == 0 ? st_hi : st_lo) + bh * D * D, n, hf, fq, c);

    // This wavefront's quarter of a K tile in LDS: chunks w4 * 64 + lane +
    // 256 e (16 bytes each) of the swizzled tile.  phi is elementwise and
    // the phi ring keeps the K layout, so a chunk converts in place of its
    // position; only the padded-key test needs the row (chunk / (D / 8)).
    constexpr int CPT = 64 * D / 8 / 256;  // chunks per thread
    const auto convert = [&](const uint16_t* kl, uint16_t* fl, int j) {
      int ct = 0, cy = 0, cx = 0;
      if (PARTIAL) cube_coords(g, j, ct, cy, cx);
      uint4 raw[CPT];
#pragma unroll
      for (int e = 0; e < CPT; ++e) raw[e] = reinterpret_cast<const uint4*>(kl)[w4 * 64 + lane + 256 * e];
#pragma unroll
      for (int e = 0; e < CPT; ++e) {
        const int p = w4 * 64 + lane + 256 * e;
        const bool valid = !PARTIAL || local_valid(g, ct, cy, cx, p / (D / 8));
        reinterpret_cast<uint4*>(fl)[p] = phi8(raw[e], valid);
      }
    };
    float dcorr = 0.f;
    bf16x8 p_prev[2] = {};
    const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
    pipeline_barrier();  // K(0) has landed
    convert(sm.k[0], sm.f[0], blk(0));
    // Step nb (u = nb % 4, as the softmax steps): after the barrier, phiK(nb)
    // is complete in f[nb % 2], K(nb+1) in k[(u+1) % 4] and V(nb-1) in
    // v[(u+3) % 4].
    auto lin_step = [&](int nb, auto uc) {
      constexpr int u = decltype(uc)::value;
      pipeline_barrier();
      bf16x8 fa[DC];
      read_k<D>(sm.f[u & 1], wk, hf, prow, fa);
      f32x16 sp = f32x16{};
#pragma unroll
      for (int dc = 0; dc < DC; ++dc) sp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[dc], fq[dc], sp, 0, 0, 0);
      bf16x8 va[DT][2];
      read_v<D>(sm.v[(u + 3) % 4], wk, hf, n, va);
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
          c[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[dt][kk], p_prev[kk], c[dt], 0, 0, 0);
      if (nb + 1 < topk) convert(sm.k[(u + 1) % 4], sm.f[(u + 1) & 1], blk(nb + 1));
      uint32_t pw[8];
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        const bf16x2 pk = __builtin_convertvector((f32x2){sp[2 * r], sp[2 * r + 1]}, bf16x2);
        dcorr = __builtin_amdgcn_fdot2_f32_bf16(pk, ones, dcorr, false);
        pw[r] = __builtin_bit_cast(uint32_t, pk) ^ 0x80008000u;  // -P' (exact in bf16)
      }
      p_prev[0] = __builtin_bit_cast(bf16x8, make_uint4(pw[0], pw[1], pw[2], pw[3]));
      p_prev[1] = __builtin_bit_cast(bf16x8, make_uint4(pw[4], pw[5], pw[6], pw[7]));
    };
    int jb = 0;
    for (; jb + 4 <= topk; jb += 4) {
      lin_step(jb, StepC<0>{});
      lin_step(jb + 1, StepC<1>{});
      lin_step(jb + 2, StepC<2>{});
      lin_step(jb + 3, StepC<3>{});
    }
    if (jb < topk) lin_step(jb, StepC<0>{});
    if (jb + 1 < topk) lin_step(jb + 1, StepC<1>{});
    if (jb + 2 < topk) lin_step(jb + 2, StepC<2>{});
    {
      pipeline_barrier();  // V(topk-1)
      bf16x8 va[DT][2];
      read_v<D>(sm.v[(topk - 1) & 3], wk, hf, n, va);
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
          c[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[dt][kk], p_prev[kk], c[dt], 0, 0, 0);
    }
    dcorr += __shfl_xor(dcorr, 32);
    __syncthreads();
    if (wk == 1) {
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) xo_lin[(dt * 16 + r) * 64 + lane] = c[dt][r];
      xd[lane] = dcorr;
    }
    __syncthreads();
    if (wk == 0) {
      const float den = (den_part + __shfl_xor(den_part, 32)) - (dcorr + xd[lane]);
      const float inv = empty_u ? 0.f : 1.f / den;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float* x = xo_lin + (dt * 16 + r) * 64 + lane;
          *x = (c[dt][r] + *x) * inv;
        }
    }
    __syncthreads();
  }
}

template <int D, bool PARTIAL>
void launch_lin_t(const KGeom& g, const uint16_t* qc, const uint16_t* kc, const uint16_t* vt, const int32_t* idx,
                  int topk, float scale, const LinTensors& lt, uint16_t* oc, float* lse, hipStream_t s) {
  const Placement pl = make_placement(g);
  attn_lin_fwd<D, PARTIAL><<<dim3(grid_size(g)), dim3(kLinThreads), 0, s>>>(
      qc, kc, vt, idx, topk, scale, scale * 1.4426950408889634f, lt.st_hi, lt.st_lo, lt.z_tot, oc, lse, g, pl);
}

}  // namespace

hipError_t launch_attn_lin_fwd(const KGeom& g, const uint16_t* qc, const uint16_t* kc, const uint16_t* vt,
                               const int32_t* idx, int topk, float scale, void* ws, uint16_t* oc, float* lse,
                               hipStream_t s) {
  // The totals only: this pass makes its phi(K) tiles itself.
  hipError_t e = launch_lin_prep(g, kc, vt, ws, s, false);
  if (e != hipSuccess) return e;
  const LinTensors lt = lin_tensors(g, ws);
  if (g.D == 64) {
    if (g.partial) launch_lin_t<64, true>(g, qc, kc, vt, idx, topk, scale, lt, oc, lse, s);
    else launch_lin_t<64, false>(g, qc, kc, vt, idx, topk, scale, lt, oc, lse, s);
  } else {
    if (g.partial) launch_lin_t<128, true>(g, qc, kc, vt, idx, topk, scale, lt, oc, lse, s);
    else launch_lin_t<128, false>(g, qc, kc, vt, idx, topk, scale, lt, oc, lse, s);
  }
  return hipGetLastError();
}

}  // namespace vsa
