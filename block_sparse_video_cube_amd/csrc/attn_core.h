// The pipelined step of the bf16 fine stage, shared by the plain fine stage
// (attn_fwd.hip) and the fine stage fused with the linear branch
// (attn_lin.hip).  See attn_fwd.hip for the design.
#pragma once

#include <math.h>

#include "tile_pipeline.h"

namespace vsa {
namespace attn_core {

using namespace tiles;

constexpr float kLazyLog2 = 8.f;

// Three K buffers (K runs two blocks ahead) and two V buffers: 80 KB at
// D = 128, so two workgroups fill the 160 KB of LDS of a compute unit.
template <int D>
struct Smem {
  uint16_t k[3][64 * D];
  uint16_t v[2][D * 64];
};

__device__ __forceinline__ float max16(const f32x16& s) {
  const float a = fmaxf(fmaxf(s[0], s[1]), s[2]), b = fmaxf(fmaxf(s[3], s[4]), s[5]);
  const float c = fmaxf(fmaxf(s[6], s[7]), s[8]), d = fmaxf(fmaxf(s[9], s[10]), s[11]);
  const float e = fmaxf(fmaxf(s[12], s[13]), s[14]);
  return fmaxf(fmaxf(fmaxf(a, b), c), fmaxf(fmaxf(d, e), s[15]));
}

// One pipelined step n.  Entering: S^T(n) (masked) in s_cur, P(n-1) in
// p_prev, and mc, the exponent offset of block n after its lazy-rescale
// decision.  The matrix cores compute S^T(n+1) = K(n+1) Q^T and
// O^T += V(n-1)^T P(n-1)^T; interleaved with them the vector units turn S^T(n)
// into P(n) = bf16(exp2(scale_log2 S^T(n) - mc)) and its row sum, then mask
// S^T(n+1) and take its per-lane max.  P is rounded once to bf16
// (v_cvt_pk_bf16_f32) and the normaliser sums the same rounded values
// (v_dot2_f32_bf16 against 1.0), so the weights applied to V sum exactly to
// the normaliser.  The tile loads of V(n) and K(n+3) go out one per MFMA slot
// of S^T(n+1); vr/kr are their buffer resources, vl/kl the LDS destinations
// of this wave's first instruction, voff/koff its lane offsets.
// PARTIAL: mask(s) masks the padded keys of S^T(n+1) (branch-free).
template <int D, bool PARTIAL, typename Mask>
__device__ __forceinline__ void step(const bf16x8 (&ka)[D / 16], const bf16x8 (&va)[D / 32][2],
                                     const bf16x8 (&qf)[D / 16], const f32x16& s_cur, f32x16& s_next,
                                     float& mx_next, const bf16x8 (&p_prev)[2], bf16x8 (&p_cur)[2],
                                     f32x16 (&o)[D / 32], float& l_run, float mc, float scale_log2,
                                     const Mask& mask, __amdgpu_buffer_rsrc_t vr, uint16_t* vl,
                                     const uint32_t* voff, __amdgpu_buffer_rsrc_t kr, uint16_t* kl,
                                     const uint32_t* koff) {
  constexpr int DC = D / 16, DT = D / 32, NI = D / 32, KRPI = 512 / D;
  constexpr int NS = DC + 2 * DT;             // MFMA slots of the step
  constexpr int NV = 48 + 10 + (PARTIAL ? 16 : 0);  // vector instructions to spread
  constexpr int VPS = (NV + NS - 1) / NS;
  static_assert(2 * NI <= DC, "one tile load per S^T slot");
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
  s_next = f32x16{};
#pragma unroll
  for (int r = 0; r < DC; ++r) {
    s_next = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[r], qf[r], s_next, 0, 0, 0);
    if (r < NI)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(vr, (lds_ptr_t)(vl + r * 8 * 64), 16, voff[r], 0, 0, 0);
    else if (r < 2 * NI)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(kr, (lds_ptr_t)(kl + (r - NI) * KRPI * D), 16, koff[r - NI], 0, 0, 0);
  }
  uint32_t pw[8];
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    const float p0 = __builtin_amdgcn_exp2f(fmaf(s_cur[2 * r], scale_log2, -mc));
    const float p1 = __builtin_amdgcn_exp2f(fmaf(s_cur[2 * r + 1], scale_log2, -mc));
    const bf16x2 pk = __builtin_convertvector((f32x2){p0, p1}, bf16x2);
    l_run = __builtin_amdgcn_fdot2_f32_bf16(pk, ones, l_run, false);
    pw[r] = __builtin_bit_cast(uint32_t, pk);
  }
  p_cur[0] = __builtin_bit_cast(bf16x8, make_uint4(pw[0], pw[1], pw[2], pw[3]));
  p_cur[1] = __builtin_bit_cast(bf16x8, make_uint4(pw[4], pw[5], pw[6], pw[7]));
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
      o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[dt][kk], p_prev[kk], o[dt], 0, 0, 0);
  if (PARTIAL) mask(s_next);
  mx_next = max16(s_next);
  // P(n) and its row sum are only used by the next step; without this the
  // compiler sinks them out of the interleaved region.
  asm volatile("" ::"v"(pw[0]), "v"(pw[1]), "v"(pw[2]), "v"(pw[3]), "v"(pw[4]), "v"(pw[5]), "v"(pw[6]), "v"(pw[7]),
               "v"(l_run));
  // S^T(n+1) first (its max closes the step), P V(n-1) after; the vector
  // work is spread evenly over all slots.
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x002, VPS, 0);
  }
}

}  // namespace attn_core
}  // namespace vsa
