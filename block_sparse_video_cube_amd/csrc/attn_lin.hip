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
// The selected part needs exactly the V tiles the fine stage streams, so here
// one workgroup of 8 wavefronts runs both on one tile pipeline:
//  * wavefronts 0-3 are the fine stage of attn_fwd.hip (same step, same
//    split: wavefront (wq, wk) owns queries 32 wq .. +31, keys 32 wk .. +31);
//  * wavefronts 4-7 take the same (wq, wk) split of phi(Q) phi(K_j)^T and
//    its product with V_j, from phi(K) tiles that run through their own ring
//    on the K schedule (phi(K) comes from lin_state, token-major, zero on
//    padded rows), and finish with phi(Q) S_tot (S_tot in bf16 hi + lo
//    halves, one per key-half wavefront) and the denominator;
//  * at the end both halves of both branches merge through LDS and the
//    wk = 0 attention wavefronts write bf16(O_sparse + O_lin) once.
// Per block the workgroup brings K, phi(K) and V tiles (48 KB at D = 128):
// 128 KB of rings, so one workgroup (two wavefronts per SIMD) per compute
// unit, where the two-call chain keeps two fine-stage workgroups per unit.
// Compared with that chain this pass saves the second read of every V tile,
// the fp32 round trip of O_sparse and a launch; it trades them for half the
// workgroups in flight to hide each query cube's prologue and epilogue.
#include <math.h>

#include "attn_core.h"

namespace vsa {

namespace {

using namespace tiles;
using namespace attn_core;

constexpr int kLinThreads = 512;

template <int D>
struct SmemL {
  uint16_t k[3][64 * D];
  uint16_t f[3][64 * D];  // phi(K) tiles, on the schedule of K
  uint16_t v[2][D * 64];
};

// One pipelined step n of a linear wavefront, mirroring step():
// S'^T(n+1) = phiK(n+1) phiQ^T on the matrix cores, P'(n) = bf16(S'^T(n)) and
// its row sum, C^T -= V(n-1)^T P'(n-1)^T (the weights enter negated, exactly);
// the loads of phiK(n+3) go out one per product slot.
template <int D>
__device__ __forceinline__ void lin_step(const bf16x8 (&fa)[D / 16], const bf16x8 (&va)[D / 32][2],
                                         const bf16x8 (&fq)[D / 16], const f32x16& s_cur, f32x16& s_next,
                                         const bf16x8 (&p_prev)[2], bf16x8 (&p_cur)[2], f32x16 (&c)[D / 32],
                                         float& dcorr, __amdgpu_buffer_rsrc_t fr, uint16_t* fl, const uint32_t* foff) {
  constexpr int DC = D / 16, DT = D / 32, NI = D / 32, KRPI = 512 / D;
  constexpr int NS = DC + 2 * DT;
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
  s_next = f32x16{};
#pragma unroll
  for (int r = 0; r < DC; ++r) {
    s_next = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[r], fq[r], s_next, 0, 0, 0);
    if (r < NI)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(fr, (lds_ptr_t)(fl + r * KRPI * D), 16, foff[r], 0, 0, 0);
  }
  uint32_t pw[8];
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    const bf16x2 pk = __builtin_convertvector((f32x2){s_cur[2 * r], s_cur[2 * r + 1]}, bf16x2);
    dcorr = __builtin_amdgcn_fdot2_f32_bf16(pk, ones, dcorr, false);
    pw[r] = __builtin_bit_cast(uint32_t, pk) ^ 0x80008000u;  // -P' (exact in bf16): C^T collects phi(Q) S_tot - sum
  }
  p_cur[0] = __builtin_bit_cast(bf16x8, make_uint4(pw[0], pw[1], pw[2], pw[3]));
  p_cur[1] = __builtin_bit_cast(bf16x8, make_uint4(pw[4], pw[5], pw[6], pw[7]));
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
      c[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[dt][kk], p_prev[kk], c[dt], 0, 0, 0);
  asm volatile("" ::"v"(pw[0]), "v"(pw[1]), "v"(pw[2]), "v"(pw[3]), "v"(pw[4]), "v"(pw[5]), "v"(pw[6]), "v"(pw[7]),
               "v"(dcorr));
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);
  }
}

template <int D, bool PARTIAL>
__global__ void __launch_bounds__(kLinThreads, 2) attn_lin_fwd(
    const uint16_t* __restrict__ qc, const uint16_t* __restrict__ kc, const uint16_t* __restrict__ vt,
    const int32_t* __restrict__ idx, int topk, float scale, float scale_log2, LinTensors lt,
    uint16_t* __restrict__ oc, float* __restrict__ lse, KGeom g, Placement pl) {
  constexpr int DC = D / 16, DT = D / 32;
  constexpr int NI = TileOffsets<D>::NI, KRPI = TileOffsets<D>::KRPI;
  constexpr int XO = DT * 16 * 64;  // floats of one wq's handed-over accumulator
  __shared__ __attribute__((aligned(16))) SmemL<D> sm;
  __shared__ float xm[2][128];  // attention wk = 1: running max and sum per query
  __shared__ float xd[2][64];   // linear wk = 1: selected-part row sum per query

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
  const TileOffsets<D> toff(w4, lane);
  const int prow = pi_row(n);
  float* xo_att = reinterpret_cast<float*>(&sm) + wq * XO;
  float* xo_lin = reinterpret_cast<float*>(&sm) + (2 + wq) * XO;

  if (role == 0) {
    // ---------------------------------------------------------------- softmax
    const uint16_t* kbase = kc + bh * g.Np * D;
    const uint16_t* vbase = vt + bh * g.Np * D;
    issue_k_tile<D>(make_rsrc(kbase + 64LL * blk(0) * D, 64 * D * 2), sm.k[0], w4, toff.k);
    bf16x8 qf[DC];
    {
      const uint16_t* qrow = qc + row * D;
#pragma unroll
      for (int dc = 0; dc < DC; ++dc) qf[dc] = *reinterpret_cast<const bf16x8*>(qrow + 16 * dc + 8 * hf);
    }
    issue_k_tile<D>(make_rsrc(kbase + 64LL * blk(1) * D, 64 * D * 2), sm.k[1], w4, toff.k);
    issue_k_tile<D>(make_rsrc(kbase + 64LL * blk(2) * D, 64 * D * 2), sm.k[2], w4, toff.k);
    {
      uint4* z = reinterpret_cast<uint4*>(sm.v[1]);  // V(-1) = 0 for both branches
#pragma unroll
      for (int e = tid; e < D * 64 * 2 / 16; e += kLinThreads / 2) z[e] = make_uint4(0, 0, 0, 0);
    }
    f32x16 o[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) o[dt] = f32x16{};
    float m_run = -INFINITY, l_run = 0.f;
    const float lazy_raw = kLazyLog2 / scale_log2;
    bf16x8 p_prev[2] = {};
    f32x16 s_cur;
    float mx_cur;
    {
      wait_vmcnt<2 * NI>();
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
    for (int jb = 0; jb < topk; jb += 6) {
#pragma unroll
      for (int u = 0; u < 6; ++u) {
        const int nb = jb + u;
        if (nb < topk) {
          wait_vmcnt<NI>();
          pipeline_barrier();
          bf16x8 ka[DC];
          bf16x8 va[DT][2];
          read_k<D>(sm.k[(u + 1) % 3], wk, hf, prow, ka);
          read_v<D>(sm.v[(u + 1) % 2], wk, hf, n, va);
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
                           [&](f32x16& s) { mask_keys(s, g, j_next, wk, hf); },
                           make_rsrc(vbase + 64LL * blk(nb) * D, 64 * D * 2),
                           sm.v[u % 2] + w4 * NI * 8 * 64, toff.v,
                           make_rsrc(kbase + 64LL * blk(nb + 3) * D, 64 * D * 2), sm.k[u % 3] + w4 * NI * KRPI * D,
                           toff.k);
          move = __builtin_amdgcn_ballot_w64(mx_next > m_run + lazy_raw) != 0;
          if (resc) {
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) o[dt] *= alpha;
          }
          s_cur = s_next;
          mx_cur = mx_next;
          p_prev[0] = p_cur[0];
          p_prev[1] = p_cur[1];
        }
      }
    }
    {
      wait_vmcnt<NI>();
      pipeline_barrier();
      bf16x8 va[DT][2];
      read_v<D>(sm.v[(topk - 1) & 1], wk, hf, n, va);
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
      xm[wq][lane] = m_run;
      xm[wq][64 + lane] = l_run;
    }
    __syncthreads();
    __syncthreads();  // the linear wavefronts have left O_lin in xo_lin
    if (wk == 1) return;
    const float m1 = xm[wq][lane], l1 = xm[wq][64 + lane];
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
    const uint16_t* fbase = lt.fk + bh * g.Np * D;
    issue_k_tile<D>(make_rsrc(fbase + 64LL * blk(0) * D, 64 * D * 2), sm.f[0], w4, toff.k);
    // phi(Q) fragments (bf16) and this lane's part of phi(Q) . z_tot.
    bf16x8 fq[DC];
    float den_part = 0.f;
    {
      const uint16_t* qrow = qc + row * D;
      const float* zt = lt.z_tot + bh * D;
#pragma unroll
      for (int dc = 0; dc < DC; ++dc) {
        const uint4 raw = *reinterpret_cast<const uint4*>(qrow + 16 * dc + 8 * hf);
        const uint32_t wv[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
        for (int e2 = 0; e2 < 4; ++e2) {
          const uint16_t p0 = f32_to_bf16(phi_elu1(__uint_as_float(wv[e2] << 16)));
          const uint16_t p1 = f32_to_bf16(phi_elu1(__uint_as_float(wv[e2] & 0xFFFF0000u)));
          fq[dc][2 * e2] = __builtin_bit_cast(__bf16, p0);
          fq[dc][2 * e2 + 1] = __builtin_bit_cast(__bf16, p1);
          const int d = 16 * dc + 8 * hf + 2 * e2;
          den_part += bf16_to_f32(p0) * zt[d] + bf16_to_f32(p1) * zt[d + 1];
        }
      }
    }
    issue_k_tile<D>(make_rsrc(fbase + 64LL * blk(1) * D, 64 * D * 2), sm.f[1], w4, toff.k);
    issue_k_tile<D>(make_rsrc(fbase + 64LL * blk(2) * D, 64 * D * 2), sm.f[2], w4, toff.k);
    // c starts as this key half's share of phi(Q) S_tot (the hi or the lo
    // half), while the first tiles arrive; the steps subtract the selected part.
    f32x16 c[DT];
    {
      const uint16_t* st = (wk == 0 ? lt.st_hi : lt.st_lo) + bh * D * D;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        c[dt] = f32x16{};
        const int e = 32 * dt + n;
#pragma unroll
        for (int dc = 0; dc < DC; ++dc) {
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(st + e * D + 16 * dc + 8 * hf);
          c[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, fq[dc], c[dt], 0, 0, 0);
        }
      }
    }
    float dcorr = 0.f;
    bf16x8 p_prev[2] = {};
    f32x16 s_cur;
    {
      wait_vmcnt<2 * NI>();
      pipeline_barrier();
      bf16x8 fa[DC];
      read_k<D>(sm.f[0], wk, hf, prow, fa);
      s_cur = f32x16{};
#pragma unroll
      for (int dc = 0; dc < DC; ++dc) s_cur = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[dc], fq[dc], s_cur, 0, 0, 0);
    }
    for (int jb = 0; jb < topk; jb += 6) {
#pragma unroll
      for (int u = 0; u < 6; ++u) {
        const int nb = jb + u;
        if (nb < topk) {
          wait_vmcnt<NI>();
          pipeline_barrier();
          bf16x8 fa[DC];
          bf16x8 va[DT][2];
          read_k<D>(sm.f[(u + 1) % 3], wk, hf, prow, fa);
          read_v<D>(sm.v[(u + 1) % 2], wk, hf, n, va);
          f32x16 s_next;
          bf16x8 p_cur[2];
          lin_step<D>(fa, va, fq, s_cur, s_next, p_prev, p_cur, c, dcorr,
                      make_rsrc(fbase + 64LL * blk(nb + 3) * D, 64 * D * 2), sm.f[u % 3] + w4 * NI * KRPI * D,
                      toff.k);
          s_cur = s_next;
          p_prev[0] = p_cur[0];
          p_prev[1] = p_cur[1];
        }
      }
    }
    {
      wait_vmcnt<NI>();
      pipeline_barrier();
      bf16x8 va[DT][2];
      read_v<D>(sm.v[(topk - 1) & 1], wk, hf, n, va);
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
          c[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[dt][kk], p_prev[kk], c[dt], 0, 0, 0);
    }
    dcorr += __shfl_xor(dcorr, 32);
    wait_vmcnt<0>();
    __syncthreads();
    if (wk == 1) {
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) xo_lin[(dt * 16 + r) * 64 + lane] = c[dt][r];
      xd[wq][lane] = dcorr;
    }
    __syncthreads();
    if (wk == 0) {
      const float den = (den_part + __shfl_xor(den_part, 32)) - (dcorr + xd[wq][lane]);
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
      qc, kc, vt, idx, topk, scale, scale * 1.4426950408889634f, lt, oc, lse, g, pl);
}

}  // namespace

hipError_t launch_attn_lin_fwd(const KGeom& g, const uint16_t* qc, const uint16_t* kc, const uint16_t* vt,
                               const int32_t* idx, int topk, float scale, void* ws, uint16_t* oc, float* lse,
                               hipStream_t s) {
  hipError_t e = launch_lin_prep(g, kc, vt, ws, s);
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
