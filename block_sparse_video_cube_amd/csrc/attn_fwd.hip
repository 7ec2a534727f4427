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
// SLOTS: packed tiles (tile_pipeline.h): K in compact cube-major rows, V in
// the slot layout [4][D][16] per cube, wavefront w loading slot w of every
// tile.  With PARTIAL the tiles come from a packing plan (block_plan: up to
// four cubes with few valid keys share a tile) and keys are masked by slot
// counts; without it every tile is one whole cube of the list.
// LIN (full tiles, cube-major K): the linear branch over the unselected cubes
// is added in the epilogue from the query cube's summed states (su: S_U^T
// rows, then z_U, as lin_unsel_sum writes them): O = O_sparse + phi(Q) S_U /
// (phi(Q) . z_U), rounded to bf16 once.
template <int D, bool PARTIAL, bool RASTER, bool KRASTER, bool SLOTS, bool LIN = false>
__global__ void __launch_bounds__(kThreads, 2) attn_fwd(const uint16_t* __restrict__ qc,
                                                        const uint16_t* __restrict__ kc,
                                                        const uint16_t* __restrict__ vt,
                                                        const int32_t* __restrict__ idx,
                                                        const int32_t* __restrict__ plan,
                                                        const int32_t* __restrict__ order, int topk, float scale,
                                                        float scale_log2, uint16_t* __restrict__ oc,
                                                        float* __restrict__ oc_f32, float* __restrict__ lse,
                                                        KGeom g, Placement pl, const uint16_t* __restrict__ su) {
  static_assert(!(SLOTS && KRASTER), "packed tiles read cube-major K");
  static_assert(!(LIN && (SLOTS || KRASTER)), "the linear epilogue runs on full tiles of cube-major K");
  constexpr bool PLAN = SLOTS && PARTIAL;
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
  // PLAN: the query cubes of a head run in the order plan_order gives
  // (most tiles first); each cube's result does not depend on that order.
  if (PLAN) i = order[bh * g.nc + i];
  // K source: the head's cube-major rows, or (RASTER) its raster rows.
  const uint16_t* kbase = KRASTER ? kc + ((long long)b * g.S * g.H + h) * D : kc + bh * g.Np * D;
  const uint16_t* vbase = vt + bh * g.Np * D;
  const int32_t* irow = idx + (bh * g.nc + i) * topk;
  // PLAN: the row of the packing plan (a header whose first word is the
  // number of tiles, then four slot codes per tile).
  const int32_t* prow = PLAN ? plan + (bh * g.nc + i) * 4LL * (topk + 1) : nullptr;
  const int ntiles = PLAN ? prow[0] : topk;
  const int q = 32 * wq + n;
  // Past the last block the pipeline keeps issuing loads (into a free buffer;
  // the K loads with a zero-size range, so they move no data) so that the
  // number of loads in flight is the same at every step.
  const auto blk = [&](int m) { return irow[m < ntiles ? m : ntiles - 1]; };
  // SLOTS: the code of slot s of tile m (tiles past the end: the last one).
  const auto slot = [&](int m, int s) {
    const int mm = m < ntiles ? m : ntiles - 1;
    return PLAN ? prow[4 * (mm + 1) + s] : ((irow[mm] << 8) | (s << 5) | 16);
  };
  // The key mask of tile m for this wavefront (PARTIAL).
  const auto mask_of = [&](int m) {
    if constexpr (SLOTS) {
      const int c0 = slot_count(slot(m, 2 * wk)), c1 = slot_count(slot(m, 2 * wk + 1));
      return [=](f32x16& s) { mask_slots(s, c0, c1, hf); };
    } else {
      const int j = blk(m);
      return [=, &g](f32x16& s) { mask_keys(s, g, j, wk, hf); };
    }
  };

  // Pipeline: K(m) lives in K buffer m % 3 and V(m) in V buffer m % 2.
  // Step n waits for K(n+1) and V(n-1), reads them, issues V(n) and K(n+3)
  // into the buffers that step n-1 finished with, and (see step) computes
  // S^T(n+1), P(n) and P(n-1) V(n-1).  V(-1) is a zero tile and P(-1) = 0.
  // Steps come in groups of six so that every buffer index is compile-time.
  const TileOffsets<D> toff(w, lane);
  uint32_t roff[NI];  // RASTER: lane offsets within a cube, and their local rows
  int rrow[NI];
  if (KRASTER) raster_lane_offsets<D>(g, w, lane, roff, rrow);
  // SLOTS: lane offsets of this wavefront's V slot (one contiguous block).
  uint32_t vso[NI];
  v_slot_offsets<D>(lane, vso);
  const uint32_t* voffs = SLOTS ? vso : toff.v;
  uint32_t kto[NI];
  // Buffer resource of this wavefront's K loads of tile m (offsets in kto).
  const auto k_rsrc = [&](int m) {
    if constexpr (SLOTS) {
#pragma unroll
      for (int e = 0; e < NI; ++e) kto[e] = toff.k[e];
      return k_slot_rsrc<D>(kbase, slot(m, w), w);
    } else {
      return k_tile_rsrc<D, PARTIAL, KRASTER>(kbase, g, blk(m), toff.k, roff, rrow, kto);
    }
  };
  // Buffer resource and LDS destination of this wavefront's V loads of tile m.
  const auto v_rsrc = [&](int m) {
    if constexpr (SLOTS) return v_slot_rsrc<D>(vbase, slot(m, w));
    else return make_rsrc(vbase + 64LL * blk(m) * D, 64 * D * 2);
  };
  const int vl_off = SLOTS ? w * 16 * D : w * NI * 8 * 64;
  {
    // V(-1) = 0.  Written before any tile load is in flight: the compiler
    // orders LDS stores after every outstanding direct-to-LDS load.
    uint4* z = reinterpret_cast<uint4*>(sm.v[1]);
#pragma unroll
    for (int e = tid; e < D * 64 * 2 / 16; e += kThreads) z[e] = make_uint4(0, 0, 0, 0);
  }
  issue_k_tile<D>(k_rsrc(0), sm.k[0], w, kto);
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
  issue_k_tile<D>(k_rsrc(1), sm.k[1], w, kto);
  issue_k_tile<D>(k_rsrc(2), sm.k[2], w, kto);
  f32x16 o[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) o[dt] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;
  const int prow_pi = pi_row(n);
  const float lazy_raw = kLazyLog2 / scale_log2;
  bf16x8 p_prev[2] = {};
  const auto read_vt = [&](const uint16_t* vlds, bf16x8 (&va)[DT][2]) {
    if constexpr (SLOTS) read_v_slots<D>(vlds, wk, hf, n, va);
    else read_v<D>(vlds, wk, hf, n, va);
  };

  f32x16 s_cur;
  float mx_cur;
  {
    // K(0) and the Q fragments are in; K(1), K(2) may stay in flight.
    wait_vmcnt<2 * NI>();
    pipeline_barrier();
    bf16x8 ka[DC];
    read_k<D>(sm.k[0], wk, hf, prow_pi, ka);
    s_cur = f32x16{};
#pragma unroll
    for (int dc = 0; dc < DC; ++dc) s_cur = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[dc], qf[dc], s_cur, 0, 0, 0);
    if (PARTIAL) mask_of(0)(s_cur);
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
    read_k<D>(sm.k[(u + 1) % 3], wk, hf, prow_pi, ka);
    read_vt(sm.v[(u + 1) % 2], va);
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
    const __amdgpu_buffer_rsrc_t krs = (nb + 3 < ntiles) ? k_rsrc(nb + 3) : make_rsrc(kbase, 0);
    step<D, PARTIAL>(ka, va, qf, s_cur, s_next, mx_next, p_prev, p_cur, o, l_run, mc, scale_log2,
                     mask_of(nb + 1), v_rsrc(nb), sm.v[u % 2] + vl_off, voffs, krs,
                     sm.k[u % 3] + w * NI * KRPI * D, kto);
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
  for (; jb + 6 <= ntiles; jb += 6) {
    run_step(jb, StepC<0>{});
    run_step(jb + 1, StepC<1>{});
    run_step(jb + 2, StepC<2>{});
    run_step(jb + 3, StepC<3>{});
    run_step(jb + 4, StepC<4>{});
    run_step(jb + 5, StepC<5>{});
  }
  if (jb < ntiles) run_step(jb, StepC<0>{});
  if (jb + 1 < ntiles) run_step(jb + 1, StepC<1>{});
  if (jb + 2 < ntiles) run_step(jb + 2, StepC<2>{});
  if (jb + 3 < ntiles) run_step(jb + 3, StepC<3>{});
  if (jb + 4 < ntiles) run_step(jb + 4, StepC<4>{});
  {
    // Last product: P(ntiles-1) V(ntiles-1).
    wait_vmcnt<NI>();
    pipeline_barrier();
    bf16x8 va[DT][2];
    read_vt(sm.v[(ntiles - 1) & 1], va);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
        o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[dt][kk], p_prev[kk], o[dt], 0, 0, 0);
  }

  // Linear branch (LIN): lin^T[e][q] = sum_d S_U^T[e][d] phi(Q)[q][d] for this
  // wavefront's half of the value dims e (tiles DT/2 wk ..), the A operands
  // straight from the query cube's S_U^T rows (eight consecutive d per lane),
  // the B operands phi(Q) from the Q fragments; the wk = 0 wavefronts also
  // form den = phi(Q) . z_U (both lane halves).
  constexpr int LT = LIN ? DT / 2 : 1;
  f32x16 lin[LT];
  float den = 0.f;
  if constexpr (LIN) {
    const uint16_t* sui = su + (bh * g.nc + i) * (long long)(D * D + D);
    bf16x8 fq[DC];
#pragma unroll
    for (int dc = 0; dc < DC; ++dc) {
      const uint4 raw = __builtin_bit_cast(uint4, qf[dc]);
      fq[dc] = __builtin_bit_cast(
          bf16x8, make_uint4(phi2_bf16(raw.x), phi2_bf16(raw.y), phi2_bf16(raw.z), phi2_bf16(raw.w)));
    }
#pragma unroll
    for (int t = 0; t < LT; ++t) {
      const int dt = wk * LT + t;
      bf16x8 a[DC];
#pragma unroll
      for (int dc = 0; dc < DC; ++dc)
        a[dc] = *reinterpret_cast<const bf16x8*>(sui + (32 * dt + n) * D + 16 * dc + 8 * hf);
      lin[t] = f32x16{};
#pragma unroll
      for (int dc = 0; dc < DC; ++dc) lin[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[dc], fq[dc], lin[t], 0, 0, 0);
    }
    if (wk == 0) {
      uint4 zr[DC];
#pragma unroll
      for (int dc = 0; dc < DC; ++dc) zr[dc] = *reinterpret_cast<const uint4*>(sui + D * D + 16 * dc + 8 * hf);
#pragma unroll
      for (int dc = 0; dc < DC; ++dc) {
        const uint4 fw = __builtin_bit_cast(uint4, fq[dc]);
        const uint32_t fa[4] = {fw.x, fw.y, fw.z, fw.w}, za[4] = {zr[dc].x, zr[dc].y, zr[dc].z, zr[dc].w};
#pragma unroll
        for (int e2 = 0; e2 < 4; ++e2)
          den = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, fa[e2]), __builtin_bit_cast(bf16x2, za[e2]),
                                                den, false);
      }
      den += __shfl_xor(den, 32);
    }
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
    if constexpr (LIN) {
      // Its value-dim tiles of the linear branch, in the second V buffer.
      float* xl = reinterpret_cast<float*>(&sm.v[1][0]) + wq * (LT * 16 * 64);
#pragma unroll
      for (int t = 0; t < LT; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) xl[(t * 16 + r) * 64 + lane] = lin[t][r];
    }
  }
  __syncthreads();
  if (wk == 1) return;
  // No unselected cube (den = 0): the linear branch is 0.
  const float inv_den = (LIN && den > 0.f) ? 1.f / den : 0.f;
  const float* xl = reinterpret_cast<const float*>(&sm.v[1][0]) + wq * (LT * 16 * 64);
  const float m1 = xm[lane], l1 = xm[64 + lane];
  const float m = fmaxf(m_run, m1);
  const float a0 = __builtin_amdgcn_exp2f((m_run - m) * scale_log2);
  const float a1 = __builtin_amdgcn_exp2f((m1 - m) * scale_log2);
  const float l_tot = l_run * a0 + l1 * a1;
  const float inv = 1.f / l_tot;
  const float c0 = a0 * inv, c1 = a1 * inv;
  const long long row = bh * g.Np + 64LL * i + q;
  // oc may be null (RASTER with only the fp32 output wanted): no pointer is formed from it then.
  uint16_t* orow = oc ? (RASTER ? oc + qtok : oc + row * D) : nullptr;
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
        if constexpr (LIN) {
          const float lv = (dt < LT) ? lin[dt < LT ? dt : 0][r] : xl[((dt - LT) * 16 + r) * 64 + lane];
          v[e] += lv * inv_den;
        }
      }
      if (qvalid && orow) *reinterpret_cast<uint2*>(orow + d) = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
      if (oc_f32) *reinterpret_cast<float4*>(oc_f32 + row * D + d) = make_float4(v[0], v[1], v[2], v[3]);
    }
  if (lse && hf == 0) lse[row] = m * scale + logf(l_tot);
}

// Packing plan of the fine stage's tiles for one list row per wavefront.  A
// selected cube with n valid keys needs ceil(n / 16) slots (compact order puts
// its valid keys first).  Cubes of three or four slots get a tile each (in
// list order), then cubes of two slots go two to a tile, then cubes of one
// slot four to a tile (each class in list order; the last tile of a class may
// have empty slots).  Row layout (int32): word 0 the number of tiles, word 1
// the mean index of the cubes that have a tile of their own (0 if none; a
// launch-order key), words 2..3 unused, then four slot codes per tile
// (tile_pipeline.h).  Positions come from ballot prefix counts: no atomics,
// the plan is deterministic.
__global__ void __launch_bounds__(256) block_plan(const int32_t* __restrict__ idx, int topk,
                                                  int32_t* __restrict__ plan, KGeom g, long long nrows) {
  const int lane = threadIdx.x & 63;
  const long long row = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= nrows) return;  // whole wavefront leaves together
  const int32_t* irow = idx + row * topk;
  int32_t* prow = plan + row * 4LL * (topk + 1);
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  const auto valid_count = [&](int j) {
    int ct, cy, cx;
    cube_coords(g, j, ct, cy, cx);
    return cube_count(g, ct, cy, cx);
  };
  int nb = 0, n2 = 0, n1 = 0;
  for (int base = 0; base < topk; base += 64) {
    const int m = base + lane;
    const int sl = m < topk ? (valid_count(irow[m]) + 15) >> 4 : 0;
    nb += __popcll(__ballot(sl >= 3));
    n2 += __popcll(__ballot(sl == 2));
    n1 += __popcll(__ballot(sl == 1));
  }
  const int t2 = (n2 + 1) >> 1, t1 = (n1 + 3) >> 2;
  const int base2 = nb, base1 = nb + t2;
  int cb = 0, c2 = 0, c1 = 0;
  unsigned own = 0;  // sum of the indices of the cubes with a tile of their own
  for (int base = 0; base < topk; base += 64) {
    const int m = base + lane;
    const int j = m < topk ? irow[m] : 0;
    const int nv = m < topk ? valid_count(j) : 0;
    const int sl = (nv + 15) >> 4;
    const uint64_t mb = __ballot(sl >= 3), m2 = __ballot(sl == 2), m1 = __ballot(sl == 1);
    const auto code = [&](int sc) {
      const int cnt = min(16, max(0, nv - 16 * sc));
      return cnt ? (j << 8) | (sc << 5) | cnt : 0;
    };
    if (sl >= 3) {
      own += j;
      const int t = cb + __popcll(mb & below);
      *reinterpret_cast<int4*>(prow + 4 * (t + 1)) = make_int4(code(0), code(1), code(2), code(3));
    } else if (sl == 2) {
      const int r = c2 + __popcll(m2 & below);
      *reinterpret_cast<int2*>(prow + 4 * (base2 + (r >> 1) + 1) + 2 * (r & 1)) = make_int2(code(0), code(1));
    } else if (sl == 1) {
      const int r = c1 + __popcll(m1 & below);
      prow[4 * (base1 + (r >> 2) + 1) + (r & 3)] = code(0);
    }
    cb += __popcll(mb);
    c2 += __popcll(m2);
    c1 += __popcll(m1);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) own += __shfl_xor(own, o);
  if (lane == 0) {
    prow[0] = nb + t2 + t1;
    prow[1] = nb ? (int)(own / (unsigned)nb) : 0;
    if (n2 & 1) *reinterpret_cast<int2*>(prow + 4 * (base2 + t2) + 2) = make_int2(0, 0);
    for (int r = n1; r < 4 * t1; ++r) prow[4 * (base1 + (r >> 2) + 1) + (r & 3)] = 0;
  }
}

// Launch order of the query cubes of each (b, h) for the packed fine stage:
// by number of tiles, most first.  Workgroups that the hardware runs together
// on an XCD (consecutive launch positions) then carry equal work, start and
// finish together, and sweep their ascending key lists in step, so tiles that
// several of them selected are fetched into the XCD's L2 once for all.
// Within equal tile counts, by the mean index of the cubes with a tile of
// their own (plan word 1), ascending and descending in turn from one tile
// count to the next, then by query cube: workgroups that run together then
// also sweep the key index range in phase, across the change of tile count
// too.  One workgroup per (b, h): the occupied tile counts in LDS, then a
// bitonic sort of (count, mean, cube) keys in LDS.  A query cube's result
// does not depend on the order.
constexpr int kOrderSortMax = 4096;  // query cubes per head sorted in LDS (32 KB of keys)

__global__ void __launch_bounds__(1024) plan_order(const int32_t* __restrict__ plan, int topk,
                                                   int32_t* __restrict__ order, int nc, int npow2) {
  extern __shared__ unsigned long long keys[];  // npow2 keys, then topk + 1 ints
  int* turn = reinterpret_cast<int*>(keys + npow2);
  const long long bh = blockIdx.x;
  const long long stride = 4LL * (topk + 1);
  const int32_t* rows = plan + bh * nc * stride;
  for (int t = threadIdx.x; t <= topk; t += 1024) turn[t] = 0;
  __syncthreads();
  for (int c = threadIdx.x; c < nc; c += 1024) atomicOr(&turn[rows[c * stride]], 1);
  __syncthreads();
  if (threadIdx.x == 0) {
    int run = 0;  // occupied tile counts from the largest down: 1 on every second one
    for (int t = topk; t >= 0; --t) {
      const int occupied = turn[t];
      turn[t] = run & 1;
      run += occupied;
    }
  }
  __syncthreads();
  for (int c = threadIdx.x; c < npow2; c += 1024) {
    unsigned long long key = ~0ull;  // padding sorts last
    if (c < nc) {
      const int2 hdr = *reinterpret_cast<const int2*>(rows + c * stride);
      const unsigned mean = turn[hdr.x] ? (unsigned)(kOrderSortMax - 1 - hdr.y) : (unsigned)hdr.y;
      key = ((unsigned long long)(topk - hdr.x) << 26) | ((unsigned long long)mean << 13) | (unsigned)c;
    }
    keys[c] = key;
  }
  __syncthreads();
  for (int k = 2; k <= npow2; k <<= 1)
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int t = threadIdx.x; t < npow2; t += 1024) {
        const int p = t ^ j;
        if (p > t) {
          const unsigned long long a = keys[t], b = keys[p];
          if ((a > b) == ((t & k) == 0)) {
            keys[t] = b;
            keys[p] = a;
          }
        }
      }
      __syncthreads();
    }
  for (int c = threadIdx.x; c < nc; c += 1024) order[bh * nc + c] = (int)(keys[c] & 0x1FFF);
}

// The same order by tile count only, for heads of more than kOrderSortMax
// query cubes: a histogram of the tile counts in LDS, bins from the largest
// count, cubes placed with LDS atomics (the order within a bin is arbitrary).
__global__ void __launch_bounds__(256) plan_order_count(const int32_t* __restrict__ plan, int topk,
                                                        int32_t* __restrict__ order, int nc) {
  extern __shared__ int bins[];  // topk + 1 counters, then the running offsets in place
  const long long bh = blockIdx.x;
  const long long stride = 4LL * (topk + 1);
  const int32_t* rows = plan + bh * nc * stride;
  for (int t = threadIdx.x; t <= topk; t += 256) bins[t] = 0;
  __syncthreads();
  for (int c = threadIdx.x; c < nc; c += 256) atomicAdd(&bins[rows[c * stride]], 1);
  __syncthreads();
  if (threadIdx.x == 0) {
    int run = 0;  // bins from the largest tile count down: exclusive offsets
    for (int t = topk; t >= 0; --t) {
      const int cnt = bins[t];
      bins[t] = run;
      run += cnt;
    }
  }
  __syncthreads();
  for (int c = threadIdx.x; c < nc; c += 256) order[bh * nc + atomicAdd(&bins[rows[c * stride]], 1)] = c;
}

template <int D, bool PARTIAL, bool RASTER, bool KRASTER, bool SLOTS = false, bool LIN = false>
void launch_fwd(const KGeom& g, const uint16_t* qc, const uint16_t* kc, const uint16_t* vt, const int32_t* idx,
                const int32_t* plan, const int32_t* order, int topk, float scale, uint16_t* oc, float* oc_f32,
                float* lse, hipStream_t s, const uint16_t* su = nullptr) {
  const Placement pl = make_placement(g);
  const float scale_log2 = scale * 1.4426950408889634f;
  attn_fwd<D, PARTIAL, RASTER, KRASTER, SLOTS, LIN><<<dim3(grid_size(g)), dim3(kThreads), 0, s>>>(
      qc, kc, vt, idx, plan, order, topk, scale, scale_log2, oc, oc_f32, lse, g, pl, su);
}

template <bool RASTER, bool KRASTER>
hipError_t launch_fwd_any(const KGeom& g, const uint16_t* q, const uint16_t* k, const uint16_t* vt,
                          const int32_t* idx, int topk, float scale, uint16_t* o, float* o_f32, float* lse,
                          hipStream_t s) {
  if (g.D == 64) {
    if (g.partial) launch_fwd<64, true, RASTER, KRASTER>(g, q, k, vt, idx, nullptr, nullptr, topk, scale, o, o_f32, lse, s);
    else launch_fwd<64, false, RASTER, KRASTER>(g, q, k, vt, idx, nullptr, nullptr, topk, scale, o, o_f32, lse, s);
  } else {
    if (g.partial) launch_fwd<128, true, RASTER, KRASTER>(g, q, k, vt, idx, nullptr, nullptr, topk, scale, o, o_f32, lse, s);
    else launch_fwd<128, false, RASTER, KRASTER>(g, q, k, vt, idx, nullptr, nullptr, topk, scale, o, o_f32, lse, s);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_fwd(const KGeom& g, const uint16_t* qc, const uint16_t* kc, const uint16_t* vt,
                           const int32_t* idx, int topk, float scale, uint16_t* oc, float* oc_f32, float* lse,
                           hipStream_t s) {
  return launch_fwd_any<false, false>(g, qc, kc, vt, idx, topk, scale, oc, oc_f32, lse, s);
}

hipError_t launch_attn_fwd_raster(const KGeom& g, const uint16_t* q, const uint16_t* k, bool k_raster,
                                  const uint16_t* vt, const int32_t* idx, int topk, float scale, uint16_t* o,
                                  float* o_f32, float* lse, hipStream_t s) {
  if (k_raster) return launch_fwd_any<true, true>(g, q, k, vt, idx, topk, scale, o, o_f32, lse, s);
  return launch_fwd_any<true, false>(g, q, k, vt, idx, topk, scale, o, o_f32, lse, s);
}

hipError_t launch_attn_fwd_linear(const KGeom& g, const uint16_t* q, bool raster, const uint16_t* kc,
                                  const uint16_t* vt, const int32_t* idx, int topk, float scale, const uint16_t* su,
                                  uint16_t* o, float* lse, hipStream_t s) {
#define VSA_LIN(DD, PP, RR) \
  launch_fwd<DD, PP, RR, false, false, true>(g, q, kc, vt, idx, nullptr, nullptr, topk, scale, o, nullptr, lse, s, su)
  if (g.D == 64) {
    if (g.partial) { if (raster) VSA_LIN(64, true, true); else VSA_LIN(64, true, false); }
    else { if (raster) VSA_LIN(64, false, true); else VSA_LIN(64, false, false); }
  } else {
    if (g.partial) { if (raster) VSA_LIN(128, true, true); else VSA_LIN(128, true, false); }
    else { if (raster) VSA_LIN(128, false, true); else VSA_LIN(128, false, false); }
  }
#undef VSA_LIN
  return hipGetLastError();
}

// Packed workspace: the plan (16 bytes per tile and a 16-byte header per
// row), then the launch order (one int32 per query cube).
size_t attn_packed_workspace_bytes(const KGeom& g, int topk) {
  if (!g.partial) return 0;
  const size_t rows = (size_t)g.B * g.H * g.nc;
  return rows * 16u * ((size_t)topk + 1) + (rows * 4u + 255) / 256 * 256;
}

hipError_t launch_packed_plan(const KGeom& g, const int32_t* idx, int topk, void* ws, hipStream_t s) {
  int32_t* plan = static_cast<int32_t*>(ws);
  const long long nrows = (long long)g.B * g.H * g.nc;
  int32_t* order = plan + nrows * 4LL * (topk + 1);
  if (g.partial) {
    block_plan<<<dim3((unsigned)((nrows + 3) / 4)), dim3(256), 0, s>>>(idx, topk, plan, g, nrows);
    if (g.nc <= kOrderSortMax) {
      int npow2 = 1;
      while (npow2 < g.nc) npow2 <<= 1;
      const size_t lds = npow2 * sizeof(unsigned long long) + (topk + 1) * sizeof(int);
      plan_order<<<dim3((unsigned)(g.B * g.H)), dim3(1024), lds, s>>>(plan, topk, order, g.nc, npow2);
    } else {
      plan_order_count<<<dim3((unsigned)(g.B * g.H)), dim3(256), (topk + 1) * sizeof(int), s>>>(plan, topk, order,
                                                                                               g.nc);
    }
  }
  return hipGetLastError();
}

hipError_t launch_attn_fwd_packed(const KGeom& g, const uint16_t* q, bool raster, const uint16_t* kc,
                                  const uint16_t* vs, const int32_t* idx, int topk, float scale, uint16_t* o,
                                  float* lse, void* ws, hipStream_t s) {
  int32_t* plan = static_cast<int32_t*>(ws);
  const long long nrows = (long long)g.B * g.H * g.nc;
  int32_t* order = plan + nrows * 4LL * (topk + 1);
  const hipError_t e = launch_packed_plan(g, idx, topk, ws, s);
  if (e != hipSuccess) return e;
#define VSA_PACKED(DD, PP, RR) \
  launch_fwd<DD, PP, RR, false, true>(g, q, kc, vs, idx, plan, order, topk, scale, o, nullptr, lse, s)
  if (g.D == 64) {
    if (g.partial) { if (raster) VSA_PACKED(64, true, true); else VSA_PACKED(64, true, false); }
    else { if (raster) VSA_PACKED(64, false, true); else VSA_PACKED(64, false, false); }
  } else {
    if (g.partial) { if (raster) VSA_PACKED(128, true, true); else VSA_PACKED(128, true, false); }
    else { if (raster) VSA_PACKED(128, false, true); else VSA_PACKED(128, false, false); }
  }
#undef VSA_PACKED
  return hipGetLastError();
}

}  // namespace vsa
