// Fine stage: block-sparse attention over the selected 64x64 cube blocks.
//
// Attention is the compute-heavy core of a video transformer (FastVideo
// attention-backend article, section on why the backend matters) and grows
// quadratically with the token count (TurboDiffusion article, section
// "稀疏、蒸馏与全链路量化"); VSA computes only the selected blocks and stays
// compatible with flash-attention style kernels (FastVideo sparse-distillation
// article, section "2. 视频稀疏注意力VSA").  This kernel is that flash-style
// pass: for every (b, h, query cube i) it streams the k selected key cubes
// and keeps an online softmax (running row max and sum) in fp32.
//
// gfx950 mapping
//  * One workgroup = one query cube = 4 wavefronts.  Wavefront (wq, wk) owns
//    query rows 32 wq .. 32 wq + 31 and key rows 32 wk .. 32 wk + 31 of every
//    selected block, so each K/V tile is read from LDS exactly once per
//    workgroup, and keeps its own online softmax over its half of the keys;
//    the two halves are merged through LDS at the end.
//  * K tile (64 x D, token-major) and V tile (D x 64, stored transposed by the
//    permute kernel) arrive by direct buffer->LDS loads
//    (buffer_load_dwordx4 ... lds) through per-tile buffer resources; K runs
//    two blocks ahead (three buffers) and V one block ahead (two buffers).  Each 16-byte chunk is placed with an
//    XOR swizzle, chosen through the global address each lane fetches, so the
//    MFMA operand reads below are free of bank conflicts.
//  * S^T = K Q^T with v_mfma_f32_32x32x16_bf16: a lane owns one query column,
//    so its row max and row sum are in-lane plus one exchange with lane ^ 32.
//    The K rows are loaded in the order pi, which makes the S^T accumulator
//    the B operand of O^T = V^T P^T directly: P never leaves registers, and
//    the per-query rescale factor of O^T is a per-lane scalar.
//  * Lazy rescaling: the running max used for the exponent only moves when a
//    new block exceeds it by more than 8 (log2 units), so P <= 2^8 and the
//    O^T rescale (a full accumulator pass) is skipped almost always.
#include <math.h>

#include "attn_core.h"

namespace vsa {

namespace {

using namespace tiles;
using namespace attn_core;

// Buffer resource and lane offsets of the K tile of cube j: the cube-major
// tile (16 KB contiguous, offsets toff), or gathered from raster rows.
template <int D, bool PARTIAL, bool RASTER>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t k_tile_rsrc(const uint16_t* kbase, const KGeom& g, int j,
                                                             const uint32_t* toff, const uint32_t* roff,
                                                             const int* rrow, uint32_t* out) {
  if (RASTER) return raster_tile<D, PARTIAL>(kbase, g, j, roff, rrow, out);
#pragma unroll
  for (int e = 0; e < D / 32; ++e) out[e] = toff[e];
  return make_rsrc(kbase + 64LL * j * D, 64 * D * 2);
}

// RASTER: Q and the output are raster-order [B, S, heads, D] instead of
// cube-major rows: Q rows are gathered into registers and output rows
// scattered back, so the layer needs no permute of Q and no unpermute.
// KRASTER (with RASTER): K is raster-order too, and its tiles are gathered row
// by row by the same direct-to-LDS loads (lane offsets from
// raster_lane_offsets, padded tokens read as zero).  V stays in the
// cube-transposed layout that the P V product reads.
template <int D, bool PARTIAL, bool RASTER, bool KRASTER>
__global__ void __launch_bounds__(kThreads, 2) attn_fwd(const uint16_t* __restrict__ qc,
                                                        const uint16_t* __restrict__ kc,
                                                        const uint16_t* __restrict__ vt,
                                                        const int32_t* __restrict__ idx, int topk, float scale,
                                                        float scale_log2, uint16_t* __restrict__ oc,
                                                        float* __restrict__ oc_f32, float* __restrict__ lse,
                                                        KGeom g, Placement pl) {
  constexpr int DC = D / 16, DT = D / 32;
  constexpr int NI = TileOffsets<D>::NI, KRPI = TileOffsets<D>::KRPI;
  __shared__ __attribute__((aligned(16))) Smem<D> sm;

  int i, h, b;
  if (!map_workgroup(g, pl, i, h, b)) return;  // whole workgroup leaves before any barrier
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wq = w & 1, wk = w >> 1;  // wave-uniform
  const int hf = lane >> 5, n = lane & 31;
  const long long bh = (long long)b * g.H + h;
  // K source: the head's cube-major rows, or (RASTER) its raster rows.
  const uint16_t* kbase = KRASTER ? kc + ((long long)b * g.S * g.H + h) * D : kc + bh * g.Np * D;
  const uint16_t* vbase = vt + bh * g.Np * D;
  const int32_t* irow = idx + (bh * g.nc + i) * topk;
  const int q = 32 * wq + n;
  // Past the last block the pipeline keeps issuing loads (into a free buffer;
  // the K loads with a zero-size range, so they move no data) so that the
  // number of loads in flight is the same at every step.
  const auto blk = [&](int m) { return irow[m < topk ? m : topk - 1]; };

  // Pipeline: K(m) lives in K buffer m % 3 and V(m) in V buffer m % 2.
  // Step n waits for K(n+1) and V(n-1), reads them, issues V(n) and K(n+3)
  // into the buffers that step n-1 finished with, and (see step) computes
  // S^T(n+1), P(n) and P(n-1) V(n-1).  V(-1) is a zero tile and P(-1) = 0.
  // Steps come in groups of six so that every buffer index is compile-time.
  const TileOffsets<D> toff(w, lane);
  uint32_t roff[NI];  // RASTER: lane offsets within a cube, and their local rows
  int rrow[NI];
  if (KRASTER) raster_lane_offsets<D>(g, w, lane, roff, rrow);
  uint32_t kto[NI];
  issue_k_tile<D>(k_tile_rsrc<D, PARTIAL, KRASTER>(kbase, g, blk(0), toff.k, roff, rrow, kto), sm.k[0], w, kto);
  // Query row q of cube i: its raster token (RASTER) and whether it is real.
  bool qvalid = true;
  long long qtok = 0;
  if (RASTER) {
    int ct, cy, cx;
    cube_coords(g, i, ct, cy, cx);
    const int t = 4 * ct + (q >> 4), y = 4 * cy + ((q >> 2) & 3), x = 4 * cx + (q & 3);
    qvalid = t < g.T && y < g.Hg && x < g.W;
    qtok = (((long long)b * g.S + ((long long)t * g.Hg + y) * g.W + x) * g.H + h) * D;
  }
  bf16x8 qf[DC];
  {
    const uint16_t* qrow = RASTER ? qc + qtok : qc + (bh * g.Np + 64LL * i + q) * D;
#pragma unroll
    for (int dc = 0; dc < DC; ++dc)
      qf[dc] = qvalid ? *reinterpret_cast<const bf16x8*>(qrow + 16 * dc + 8 * hf) : bf16x8{};
  }
  issue_k_tile<D>(k_tile_rsrc<D, PARTIAL, KRASTER>(kbase, g, blk(1), toff.k, roff, rrow, kto), sm.k[1], w, kto);
  issue_k_tile<D>(k_tile_rsrc<D, PARTIAL, KRASTER>(kbase, g, blk(2), toff.k, roff, rrow, kto), sm.k[2], w, kto);
  {
    uint4* z = reinterpret_cast<uint4*>(sm.v[1]);
#pragma unroll
    for (int e = tid; e < D * 64 * 2 / 16; e += kThreads) z[e] = make_uint4(0, 0, 0, 0);
  }
  f32x16 o[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) o[dt] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;
  const int prow = pi_row(n);
  const float lazy_raw = kLazyLog2 / scale_log2;
  bf16x8 p_prev[2] = {};

  f32x16 s_cur;
  float mx_cur;
  {
    // K(0) and the Q fragments are in; K(1), K(2) may stay in flight.
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
  // Lazy rescaling: the reference max m_run moves only when a block exceeds
  // it by more than kLazyLog2 (log2 units), so P <= 2^8 and the O^T rescale
  // (a full accumulator pass) is rare.  Each lane half's max bounds the row
  // max from below, so the move is first detected per half and only then is
  // the row max taken across lane ^ 32.  A half holding padded keys only
  // (max -inf) never triggers it.
  bool move = __builtin_amdgcn_ballot_w64(mx_cur > m_run + lazy_raw) != 0;

  // One step, u = nb % 6 (compile-time).  Full groups of six steps run
  // without a per-step guard, so the values a step hands to the next (S^T,
  // its max, P) stay in place instead of being copied where a guarded step
  // would rejoin; at most five guarded steps finish the list.
  auto run_step = [&](int nb, auto uc) {
    constexpr int u = decltype(uc)::value;
    // Outstanding, oldest first: K(nb+1), V(nb-1), K(nb+2).
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
    // Until a valid key has been seen every logit is -inf and p must be 0.
    const float mc = (m_run == -INFINITY) ? 0.f : m_run * scale_log2;
    f32x16 s_next;
    float mx_next;
    bf16x8 p_cur[2];
    // Past the last block the padding loads target a zero-size range: no memory traffic.
    const __amdgpu_buffer_rsrc_t krs = (nb + 3 < topk)
        ? k_tile_rsrc<D, PARTIAL, KRASTER>(kbase, g, blk(nb + 3), toff.k, roff, rrow, kto)
        : make_rsrc(kbase, 0);
    step<D, PARTIAL>(ka, va, qf, s_cur, s_next, mx_next, p_prev, p_cur, o, l_run, mc, scale_log2, g,
                     blk(nb + 1), wk, hf, make_rsrc(vbase + 64LL * blk(nb) * D, 64 * D * 2),
                     sm.v[u % 2] + w * NI * 8 * 64, toff.v, krs, sm.k[u % 3] + w * NI * KRPI * D, kto);
    move = __builtin_amdgcn_ballot_w64(mx_next > m_run + lazy_raw) != 0;
    if (resc) {
      // O^T now holds P(0..n-1) V at the previous reference max.
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) o[dt] *= alpha;
    }
    s_cur = s_next;
    mx_cur = mx_next;
    p_prev[0] = p_cur[0];
    p_prev[1] = p_cur[1];
  };
  int jb = 0;
  for (; jb + 6 <= topk; jb += 6) {
    run_step(jb, StepC<0>{});
    run_step(jb + 1, StepC<1>{});
    run_step(jb + 2, StepC<2>{});
    run_step(jb + 3, StepC<3>{});
    run_step(jb + 4, StepC<4>{});
    run_step(jb + 5, StepC<5>{});
  }
  if (jb < topk) run_step(jb, StepC<0>{});
  if (jb + 1 < topk) run_step(jb + 1, StepC<1>{});
  if (jb + 2 < topk) run_step(jb + 2, StepC<2>{});
  if (jb + 3 < topk) run_step(jb + 3, StepC<3>{});
  if (jb + 4 < topk) run_step(jb + 4, StepC<4>{});
  {
    // Last product: P(topk-1) V(topk-1).
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

  // Merge the two key halves: wavefronts with wk = 1 hand (m, l, O^T) over.
  l_run += __shfl_xor(l_run, 32);
  wait_vmcnt<0>();  // the padding loads past the end target the K buffers
  __syncthreads();  // all LDS tile reads done; reuse the K buffers
  float* xo = reinterpret_cast<float*>(&sm.k[0][0]) + wq * (DT * 16 * 64);
  float* xm = reinterpret_cast<float*>(&sm.v[0][0]) + wq * 128;
  if (wk == 1) {
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) xo[(dt * 16 + r) * 64 + lane] = o[dt][r];
    xm[lane] = m_run;
    xm[64 + lane] = l_run;
  }
  __syncthreads();
  if (wk == 1) return;
  const float m1 = xm[lane], l1 = xm[64 + lane];
  const float m = fmaxf(m_run, m1);
  const float a0 = __builtin_amdgcn_exp2f((m_run - m) * scale_log2);
  const float a1 = __builtin_amdgcn_exp2f((m1 - m) * scale_log2);
  const float l_tot = l_run * a0 + l1 * a1;
  const float inv = 1.f / l_tot;
  const float c0 = a0 * inv, c1 = a1 * inv;
  const long long row = bh * g.Np + 64LL * i + q;
  uint16_t* orow = RASTER ? oc + qtok : oc + row * D;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int gq = 0; gq < 4; ++gq) {
      const int d = 32 * dt + 8 * gq + 4 * hf;
      float v[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 4 * gq + e;
        v[e] = o[dt][r] * c0 + xo[(dt * 16 + r) * 64 + lane] * c1;
      }
      if (qvalid) *reinterpret_cast<uint2*>(orow + d) = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
      if (!RASTER && oc_f32) *reinterpret_cast<float4*>(oc_f32 + row * D + d) = make_float4(v[0], v[1], v[2], v[3]);
    }
  if (lse && hf == 0) lse[row] = m * scale + logf(l_tot);
}

}  // namespace

template <int D, bool PARTIAL, bool RASTER, bool KRASTER>
void launch_fwd(const KGeom& g, const uint16_t* qc, const uint16_t* kc, const uint16_t* vt, const int32_t* idx,
                int topk, float scale, uint16_t* oc, float* oc_f32, float* lse, hipStream_t s) {
  const Placement pl = make_placement(g);
  const float scale_log2 = scale * 1.4426950408889634f;
  attn_fwd<D, PARTIAL, RASTER, KRASTER><<<dim3(grid_size(g)), dim3(kThreads), 0, s>>>(
      qc, kc, vt, idx, topk, scale, scale_log2, oc, oc_f32, lse, g, pl);
}

template <bool RASTER, bool KRASTER>
hipError_t launch_fwd_any(const KGeom& g, const uint16_t* q, const uint16_t* k, const uint16_t* vt,
                          const int32_t* idx, int topk, float scale, uint16_t* o, float* o_f32, float* lse,
                          hipStream_t s) {
  if (g.D == 64) {
    if (g.partial) launch_fwd<64, true, RASTER, KRASTER>(g, q, k, vt, idx, topk, scale, o, o_f32, lse, s);
    else launch_fwd<64, false, RASTER, KRASTER>(g, q, k, vt, idx, topk, scale, o, o_f32, lse, s);
  } else {
    if (g.partial) launch_fwd<128, true, RASTER, KRASTER>(g, q, k, vt, idx, topk, scale, o, o_f32, lse, s);
    else launch_fwd<128, false, RASTER, KRASTER>(g, q, k, vt, idx, topk, scale, o, o_f32, lse, s);
  }
  return hipGetLastError();
}

hipError_t launch_attn_fwd(const KGeom& g, const uint16_t* qc, const uint16_t* kc, const uint16_t* vt,
                           const int32_t* idx, int topk, float scale, uint16_t* oc, float* oc_f32, float* lse,
                           hipStream_t s) {
  return launch_fwd_any<false, false>(g, qc, kc, vt, idx, topk, scale, oc, oc_f32, lse, s);
}

hipError_t launch_attn_fwd_raster(const KGeom& g, const uint16_t* q, const uint16_t* k, bool k_raster,
                                  const uint16_t* vt, const int32_t* idx, int topk, float scale, uint16_t* o,
                                  float* lse, hipStream_t s) {
  if (k_raster) return launch_fwd_any<true, true>(g, q, k, vt, idx, topk, scale, o, nullptr, lse, s);
  return launch_fwd_any<true, false>(g, q, k, vt, idx, topk, scale, o, nullptr, lse, s);
}

}  // namespace vsa
