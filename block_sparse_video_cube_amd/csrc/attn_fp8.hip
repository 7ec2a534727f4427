// Low-precision fine stage: block-sparse attention with fp8 (E4M3) matrix
// products, after the 8-bit attention of SageAttention that TurboDiffusion
// builds its sparse-linear attention on (TurboDiffusion article, section
// "稀疏、蒸馏与全链路量化": the key matrix products at 8 bits or lower, and
// sparsity orthogonal to low-bit matrix cores).
//
// Inputs (quant.hip): Q and K codes per (b, h, cube) scale, V^T codes per
// (b, h, channel) scale over the head.  For query cube i and key cube j,
//   logits = scale * sq_i * sk_j * (Q8 K8^T),
// the online softmax runs in fp32 as in the bf16 fine stage, P (scaled so that
// a row's largest weight lies in [2^4, 2^8], inside E4M3's range) is rounded to
// E4M3, and
//   O = sv * (V8^T P8^T) / (1^T P8^T),
// with the normaliser summing exactly the rounded weights: it is a ones row
// appended to V8^T in the same matrix product.
//
// gfx950 mapping
//  * v_mfma_f32_32x32x64_f8f6f4: lanes l and l + 32 hold the two 32-byte
//    halves (32 k values each) of row / column l % 32 of the A / B operand.
//  * One workgroup = one query cube = 2 wavefronts; wavefront wq owns queries
//    32 wq .. 32 wq + 31 and all 64 keys of each block, so no merge across
//    wavefronts is needed.  S^T = K Q^T is two 32-key tiles (keys read in pi
//    order, as in the bf16 stage), each two K=64 products over D = 128.
//  * P^T of both tiles packs into one 32-byte B operand per lane (tile 0's 16
//    values, then tile 1's), which is why V^T is stored with its keys in that
//    order (vkey_pos in quant.hip): O^T += V^T P^T is one product per
//    32-channel tile, plus one for the ones row.
//  * fp8 tiles are 8 KB at D = 128: K three blocks deep and V two, 40 KB per
//    workgroup, four workgroups (eight wavefronts) per compute unit.
#include <math.h>

#include "tile_pipeline.h"

namespace vsa {

namespace {

using namespace tiles;
typedef int i32x8 __attribute__((ext_vector_type(8)));
constexpr int kThreads8 = 128;
// Lazy rescale by more than 2^4 only, and weights scaled by 2^4: the largest
// weight of a row stays in [2^4, 2^8] (E4M3 reaches 448), far above the
// subnormal range (< 2^-6) where small weights would lose their precision.
constexpr float kLazy8 = 4.f;
constexpr float kShift8 = 4.f;

__device__ __forceinline__ f32x16 mfma8(const i32x8& a, const i32x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// LDS tiles.  K: 64 rows x D bytes, 16-byte chunks swizzled by the row
// (row % (D / 16)).  V^T: D rows x 64 bytes, chunks swizzled by (row / 4) % 4.
template <int D>
struct Smem8 {
  uint8_t k[3][64 * D];
  uint8_t v[2][D * 64];
};

template <int D>
__device__ __forceinline__ int k8_chunk(int row, int chunk) {
  return chunk ^ (row & (D / 16 - 1));
}
__device__ __forceinline__ int v8_chunk(int row, int chunk) { return chunk ^ ((row >> 2) & 3); }

// Lane offsets of this wave's share of a K or V^T tile load (64 D bytes =
// D / 16 instructions of 1 KB, D / 32 per wave).
template <int D>
struct Offsets8 {
  static constexpr int NI = D / 32;
  uint32_t k[NI], v[NI];
  __device__ __forceinline__ Offsets8(int w, int lane) {
    constexpr int KCH = D / 16;        // 16-byte chunks per K row
    constexpr int KR = 1024 / D;       // K rows per instruction
#pragma unroll
    for (int e = 0; e < NI; ++e) {
      const int kr = (w * NI + e) * KR + lane / KCH;
      k[e] = (uint32_t)(kr * D + k8_chunk<D>(kr, lane % KCH) * 16);
      const int vr = (w * NI + e) * 16 + lane / 4;  // 16 V^T rows of 64 bytes per instruction
      v[e] = (uint32_t)(vr * 64 + v8_chunk(vr, lane % 4) * 16);
    }
  }
};

template <int D>
__device__ __forceinline__ void issue8(__amdgpu_buffer_rsrc_t r, uint8_t* lds, int w, const uint32_t* off) {
  constexpr int NI = D / 32;
#pragma unroll
  for (int e = 0; e < NI; ++e)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)(lds + (w * NI + e) * 1024), 16, off[e], 0, 0, 0);
}

// A operand of S^T: 32 K rows of tile t (rows 32 t + pi(m)), 32 bytes of
// channels 64 c + 32 hf .. + 31 for each of the D / 64 products.
template <int D>
__device__ __forceinline__ void read_k8(const uint8_t* lds, int t, int hf, int prow, i32x8 (&ka)[D / 64]) {
  const int row = 32 * t + prow;
#pragma unroll
  for (int c = 0; c < D / 64; ++c) {
    const int ch = 4 * c + 2 * hf;
    const uint4 a = *reinterpret_cast<const uint4*>(lds + row * D + k8_chunk<D>(row, ch) * 16);
    const uint4 b = *reinterpret_cast<const uint4*>(lds + row * D + k8_chunk<D>(row, ch + 1) * 16);
    ka[c] = i32x8{(int)a.x, (int)a.y, (int)a.z, (int)a.w, (int)b.x, (int)b.y, (int)b.z, (int)b.w};
  }
}

// A operand of O^T: channel rows 32 dt + n, the 32 key bytes of lane half hf.
template <int D>
__device__ __forceinline__ void read_v8(const uint8_t* lds, int hf, int n, i32x8 (&va)[D / 32]) {
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) {
    const int row = 32 * dt + n;
    const uint4 a = *reinterpret_cast<const uint4*>(lds + row * 64 + v8_chunk(row, 2 * hf) * 16);
    const uint4 b = *reinterpret_cast<const uint4*>(lds + row * 64 + v8_chunk(row, 2 * hf + 1) * 16);
    va[dt] = i32x8{(int)a.x, (int)a.y, (int)a.z, (int)a.w, (int)b.x, (int)b.y, (int)b.z, (int)b.w};
  }
}

// Largest of 32 values as a tree of three-input maxima (v_max3_f32).
__device__ __forceinline__ float max32(const f32x16& a, const f32x16& b) {
  float m[8];
#pragma unroll
  for (int r = 0; r < 8; ++r) m[r] = fmaxf(fmaxf(a[2 * r], a[2 * r + 1]), fmaxf(b[2 * r], b[2 * r + 1]));
  const float x = fmaxf(fmaxf(m[0], m[1]), m[2]), y = fmaxf(fmaxf(m[3], m[4]), m[5]);
  return fmaxf(fmaxf(x, y), fmaxf(m[6], m[7]));
}

// Four fp32 P values -> four E4M3 codes (P <= 2^8 < 448 needs no clamp).
__device__ __forceinline__ int pack_p(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  return __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
}

// One pipelined step n (as the bf16 stage): S^T(n+1) on the matrix cores
// with the softmax of block n and P(n-1) V(n-1); tile loads of V(n), K(n+3).
template <int D, bool PARTIAL>
__device__ __forceinline__ void step8(const i32x8 (&ka)[2][D / 64], const uint8_t* v_lds, int n, const i32x8& ones,
                                      const i32x8 (&qf)[D / 64], const f32x16 (&s_cur)[2], f32x16 (&s_next)[2],
                                      float& mx_next, const i32x8& p_prev, i32x8& p_cur, f32x16 (&o)[D / 32 + 1],
                                      float c_cur, float mc, const KGeom& g, int j_next, int hf,
                                      __amdgpu_buffer_rsrc_t vr, uint8_t* vl, const uint32_t* voff,
                                      __amdgpu_buffer_rsrc_t kr, uint8_t* kl, const uint32_t* koff) {
  constexpr int DC = D / 64, DT = D / 32, NI = D / 32;
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    s_next[t] = f32x16{};
#pragma unroll
    for (int c = 0; c < DC; ++c) s_next[t] = mfma8(ka[t][c], qf[c], s_next[t]);
    // The V tile's loads after the first key tile's products, the K tile's after the second.
#pragma unroll
    for (int e = 0; e < NI; ++e) {
      if (t == 0)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(vr, (lds_ptr_t)(vl + e * 1024), 16, voff[e], 0, 0, 0);
      else
        __builtin_amdgcn_raw_ptr_buffer_load_lds(kr, (lds_ptr_t)(kl + e * 1024), 16, koff[e], 0, 0, 0);
    }
  }
  // V^T(n-1) operands only now, in the registers the K operands held.
  i32x8 va[DT];
  read_v8<D>(v_lds, hf, n, va);
  int pw[8];
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      float p[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) p[e] = __builtin_amdgcn_exp2f(fmaf(s_cur[t][4 * r4 + e], c_cur, -mc));
      pw[4 * t + r4] = pack_p(p[0], p[1], p[2], p[3]);
    }
  p_cur = i32x8{pw[0], pw[1], pw[2], pw[3], pw[4], pw[5], pw[6], pw[7]};
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) o[dt] = mfma8(va[dt], p_prev, o[dt]);
  o[DT] = mfma8(ones, p_prev, o[DT]);
  if (PARTIAL) {
    mask_keys(s_next[0], g, j_next, 0, hf);
    mask_keys(s_next[1], g, j_next, 1, hf);
  }
  mx_next = max32(s_next[0], s_next[1]);
  asm volatile("" ::"v"(pw[0]), "v"(pw[1]), "v"(pw[2]), "v"(pw[3]), "v"(pw[4]), "v"(pw[5]), "v"(pw[6]),
               "v"(pw[7]));
  // The first 32 vector instructions (the softmax of block n, which needs
  // only S^T(n)) go ahead while the K operands of the first product arrive
  // from LDS; then the matrix products one at a time with eight vector
  // instructions between, the V^T operand reads after the first key tile's
  // products.  (Measured: about 11 % faster than starting with a product.)
  __builtin_amdgcn_sched_group_barrier(0x002, 32, 0);
#pragma unroll
  for (int s = 0; s < 2 * DC + DT + 1; ++s) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x002, 8, 0);
    if (s == DC - 1) __builtin_amdgcn_sched_group_barrier(0x100, 2 * DT, 0);
  }
}

// RASTER: the output is written in raster order [B, S, heads, D] (padded
// query rows skipped) instead of cube-major rows.
template <int D, bool PARTIAL, bool RASTER>
__global__ void __launch_bounds__(kThreads8, 2) attn_fwd_fp8(const uint8_t* __restrict__ q8,
                                                              const float* __restrict__ qscale,
                                                              const uint8_t* __restrict__ k8,
                                                              const float* __restrict__ kscale,
                                                              const uint8_t* __restrict__ v8t,
                                                              const float* __restrict__ vscale,
                                                              const int32_t* __restrict__ idx, int topk,
                                                              float scale_log2, uint16_t* __restrict__ oc,
                                                              float* __restrict__ lse, KGeom g, Placement pl) {
  constexpr int DC = D / 64, DT = D / 32, NI8 = D / 32;
  __shared__ __attribute__((aligned(16))) Smem8<D> sm;
  int i, h, b;
  if (!map_workgroup(g, pl, i, h, b)) return;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wq = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hf = lane >> 5, n = lane & 31;
  const long long bh = (long long)b * g.H + h;
  const uint8_t* kbase = k8 + bh * g.Np * D;
  const uint8_t* vbase = v8t + bh * g.Np * D;
  const float* ks = kscale + bh * g.nc;
  const int32_t* irow = idx + (bh * g.nc + i) * topk;
  const int q = 32 * wq + n;
  const auto blk = [&](int m) { return irow[m < topk ? m : topk - 1]; };
  // Per-block logit multiplier scale * log2(e) * sq_i * sk_j, kept above 0 so
  // that masked (-inf) logits stay -inf when a cube is all zero (scale 0).
  const float c_q = scale_log2 * qscale[bh * g.nc + i];
  const auto cblk = [&](int j) { return fmaxf(c_q * ks[j], 1e-30f); };
  const Offsets8<D> off(wq, lane);

  issue8<D>(make_rsrc(kbase + 64LL * blk(0) * D, 64 * D), sm.k[0], wq, off.k);
  i32x8 qf[DC];
  {
    const uint8_t* qrow = q8 + (bh * g.Np + 64LL * i + q) * D;
#pragma unroll
    for (int c = 0; c < DC; ++c) {
      const uint4 a = *reinterpret_cast<const uint4*>(qrow + 64 * c + 32 * hf);
      const uint4 bb = *reinterpret_cast<const uint4*>(qrow + 64 * c + 32 * hf + 16);
      qf[c] = i32x8{(int)a.x, (int)a.y, (int)a.z, (int)a.w, (int)bb.x, (int)bb.y, (int)bb.z, (int)bb.w};
    }
  }
  issue8<D>(make_rsrc(kbase + 64LL * blk(1) * D, 64 * D), sm.k[1], wq, off.k);
  issue8<D>(make_rsrc(kbase + 64LL * blk(2) * D, 64 * D), sm.k[2], wq, off.k);
  {
    uint4* z = reinterpret_cast<uint4*>(sm.v[1]);  // V(-1) = 0
    for (int e = tid; e < D * 64 / 16; e += kThreads8) z[e] = make_uint4(0, 0, 0, 0);
  }
  // Ones row of the normaliser: row 0 of an extra 32-row A operand.
  const int one = (n == 0) ? 0x38383838 : 0;  // four E4M3 ones
  const i32x8 ones = {one, one, one, one, one, one, one, one};
  f32x16 o[DT + 1];
#pragma unroll
  for (int dt = 0; dt <= DT; ++dt) o[dt] = f32x16{};
  float m_run = -INFINITY;  // running max, log2 units of the scaled logits
  const int prow = pi_row(n);
  i32x8 p_prev = {};

  f32x16 s_cur[2];
  float c_cur;
  float mx_cur;
  {
    wait_vmcnt<2 * NI8>();  // K(0) and Q in; K(1), K(2) may stay in flight
    pipeline_barrier();
    i32x8 ka[2][DC];
    read_k8<D>(sm.k[0], 0, hf, prow, ka[0]);
    read_k8<D>(sm.k[0], 1, hf, prow, ka[1]);
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      s_cur[t] = f32x16{};
#pragma unroll
      for (int c = 0; c < DC; ++c) s_cur[t] = mfma8(ka[t][c], qf[c], s_cur[t]);
    }
    if (PARTIAL) {
      mask_keys(s_cur[0], g, blk(0), 0, hf);
      mask_keys(s_cur[1], g, blk(0), 1, hf);
    }
    c_cur = cblk(blk(0));
    mx_cur = max32(s_cur[0], s_cur[1]) * c_cur;
  }
  bool move = __builtin_amdgcn_ballot_w64(mx_cur > m_run + kLazy8) != 0;

  // One step, u = nb % 6 (compile-time).  Full groups of six steps run
  // without a per-step guard, so the values a step hands to the next stay in
  // place instead of being copied where a guarded step would rejoin; at most
  // five guarded steps finish the list.
  auto run_step = [&](int nb, auto uc) {
    constexpr int u = decltype(uc)::value;
    wait_vmcnt<NI8>();  // K(nb+1), V(nb-1) in; K(nb+2) may stay in flight
    pipeline_barrier();
    i32x8 ka[2][DC];
    read_k8<D>(sm.k[(u + 1) % 3], 0, hf, prow, ka[0]);
    read_k8<D>(sm.k[(u + 1) % 3], 1, hf, prow, ka[1]);
    float alpha = 1.f;
    const bool resc = move;
    if (resc) {
      const float row_max = fmaxf(mx_cur, __shfl_xor(mx_cur, 32));
      const bool grow = row_max > m_run + kLazy8;
      alpha = grow ? __builtin_amdgcn_exp2f(m_run - row_max) : 1.f;
      m_run = grow ? row_max : m_run;
    }
    const float mc = (m_run == -INFINITY) ? 0.f : m_run - kShift8;
    const int j_next = blk(nb + 1);
    const float c_next = cblk(j_next);
    f32x16 s_next[2];
    float mx_next;
    i32x8 p_cur;
    // Past the last block the padding loads of K target a zero-size range: no memory traffic.
    step8<D, PARTIAL>(ka, sm.v[(u + 1) % 2], n, ones, qf, s_cur, s_next, mx_next, p_prev, p_cur, o, c_cur, mc, g, j_next, hf,
                      make_rsrc(vbase + 64LL * blk(nb) * D, 64 * D), sm.v[u % 2] + wq * NI8 * 1024, off.v,
                      (nb + 3 < topk ? make_rsrc(kbase + 64LL * blk(nb + 3) * D, 64 * D) : make_rsrc(kbase, 0)), sm.k[u % 3] + wq * NI8 * 1024,
                      off.k);
    mx_next *= c_next;
    move = __builtin_amdgcn_ballot_w64(mx_next > m_run + kLazy8) != 0;
    if (resc) {
#pragma unroll
      for (int dt = 0; dt <= DT; ++dt) o[dt] *= alpha;
    }
    s_cur[0] = s_next[0];
    s_cur[1] = s_next[1];
    c_cur = c_next;
    mx_cur = mx_next;
    p_prev = p_cur;
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
    wait_vmcnt<NI8>();
    pipeline_barrier();
    i32x8 va[DT];
    read_v8<D>(sm.v[(topk - 1) & 1], hf, n, va);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) o[dt] = mfma8(va[dt], p_prev, o[dt]);
    o[DT] = mfma8(ones, p_prev, o[DT]);
  }
  wait_vmcnt<0>();

  // Row 0 of the ones tile (register 0 of lane half 0) is the normaliser of
  // query column n.
  const float l_q = __shfl(o[DT][0], n);
  const float inv = 1.f / l_q;
  const long long row = bh * g.Np + 64LL * i + q;
  const float* vs = vscale + bh * D;
  uint16_t* orow = oc + row * D;
  bool qvalid = true;
  if (RASTER) {
    int ct, cy, cx;
    cube_coords(g, i, ct, cy, cx);
    const int t = 4 * ct + (q >> 4), y = 4 * cy + ((q >> 2) & 3), x = 4 * cx + (q & 3);
    qvalid = t < g.T && y < g.Hg && x < g.W;
    orow = oc + (((long long)b * g.S + ((long long)t * g.Hg + y) * g.W + x) * g.H + h) * D;
  }
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int gq = 0; gq < 4; ++gq) {
      const int d = 32 * dt + 8 * gq + 4 * hf;
      const f32x4 s4 = *reinterpret_cast<const f32x4*>(vs + d);
      float v[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = o[dt][4 * gq + e] * s4[e] * inv;
      if (qvalid) *reinterpret_cast<uint2*>(orow + d) = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
    }
  // m_run is in log2 units of the scaled logits, the weights carry 2^kShift8;
  // lse in natural units.
  if (lse && hf == 0) lse[row] = (m_run - kShift8) * 0.6931471805599453f + logf(l_q);
}

}  // namespace

template <int D, bool PARTIAL, bool RASTER>
static void launch_fp8_t(const KGeom& g, const uint8_t* q8, const float* qs, const uint8_t* k8, const float* ks,
                         const uint8_t* v8t, const float* vs, const int32_t* idx, int topk, float scale,
                         uint16_t* oc, float* lse, hipStream_t s) {
  const Placement pl = make_placement(g);
  attn_fwd_fp8<D, PARTIAL, RASTER><<<dim3(grid_size(g)), dim3(kThreads8), 0, s>>>(
      q8, qs, k8, ks, v8t, vs, idx, topk, scale * 1.4426950408889634f, oc, lse, g, pl);
}

template <bool RASTER>
static void launch_fp8_any(const KGeom& g, const uint8_t* q8, const float* qs, const uint8_t* k8, const float* ks,
                           const uint8_t* v8t, const float* vs, const int32_t* idx, int topk, float scale,
                           uint16_t* oc, float* lse, hipStream_t s) {
  if (g.D == 64) {
    if (g.partial) launch_fp8_t<64, true, RASTER>(g, q8, qs, k8, ks, v8t, vs, idx, topk, scale, oc, lse, s);
    else launch_fp8_t<64, false, RASTER>(g, q8, qs, k8, ks, v8t, vs, idx, topk, scale, oc, lse, s);
  } else {
    if (g.partial) launch_fp8_t<128, true, RASTER>(g, q8, qs, k8, ks, v8t, vs, idx, topk, scale, oc, lse, s);
    else launch_fp8_t<128, false, RASTER>(g, q8, qs, k8, ks, v8t, vs, idx, topk, scale, oc, lse, s);
  }
}

hipError_t launch_attn_fwd_fp8(const KGeom& g, const uint8_t* q8, const float* qs, const uint8_t* k8,
                               const float* ks, const uint8_t* v8t, const float* vs, const int32_t* idx, int topk,
                               float scale, bool raster_out, uint16_t* o, float* lse, hipStream_t s) {
  if (raster_out) launch_fp8_any<true>(g, q8, qs, k8, ks, v8t, vs, idx, topk, scale, o, lse, s);
  else launch_fp8_any<false>(g, q8, qs, k8, ks, v8t, vs, idx, topk, scale, o, lse, s);
  return hipGetLastError();
}

}  // namespace vsa
