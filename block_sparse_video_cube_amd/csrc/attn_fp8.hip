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

// This wavefront's share of a K or V^T tile load: D / 32 instructions of
// 1 KB; instruction e covers 1024 / D rows of the tile (K) and uses r[64 e / D]
// (two resources: the two slots of the wavefront's K rows with packed tiles,
// else the same one twice).
template <int D>
__device__ __forceinline__ void issue8s(const __amdgpu_buffer_rsrc_t (&r)[2], uint8_t* lds, int w,
                                        const uint32_t* off) {
  constexpr int NI = D / 32;
#pragma unroll
  for (int e = 0; e < NI; ++e)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r[(64 * e) / D], (lds_ptr_t)(lds + (w * NI + e) * 1024), 16, off[e], 0,
                                             0, 0);
}

// A operand of S^T: 32 K rows of tile t (rows 32 t + pi(m)), 32 bytes of
// channels 64 c + 32 hf .. + 31 for each of the D / 64 products.
template <int D>
__device__ __forceinline__ void read_k8(const uint8_t* __restrict__ lds, int t, int hf, int prow, i32x8 (&ka)[D / 64]) {
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
__device__ __forceinline__ void read_v8(const uint8_t* __restrict__ lds, int hf, int n, i32x8 (&va)[D / 32]) {
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) {
    const int row = 32 * dt + n;
    const uint4 a = *reinterpret_cast<const uint4*>(lds + row * 64 + v8_chunk(row, 2 * hf) * 16);
    const uint4 b = *reinterpret_cast<const uint4*>(lds + row * 64 + v8_chunk(row, 2 * hf + 1) * 16);
    va[dt] = i32x8{(int)a.x, (int)a.y, (int)a.z, (int)a.w, (int)b.x, (int)b.y, (int)b.z, (int)b.w};
  }
}

// Largest of 32 values as chains of three-input maxima (v_max3_f32).
__device__ __forceinline__ float max32(const f32x16& a, const f32x16& b) {
  const float x = fmaxf(fmaxf(a[0], a[1]), a[2]), y = fmaxf(fmaxf(a[3], a[4]), a[5]);
  const float z = fmaxf(fmaxf(a[6], a[7]), a[8]), u = fmaxf(fmaxf(a[9], a[10]), a[11]);
  const float v = fmaxf(fmaxf(a[12], a[13]), a[14]), w = fmaxf(fmaxf(a[15], b[0]), b[1]);
  const float x2 = fmaxf(fmaxf(b[2], b[3]), b[4]), y2 = fmaxf(fmaxf(b[5], b[6]), b[7]);
  const float z2 = fmaxf(fmaxf(b[8], b[9]), b[10]), u2 = fmaxf(fmaxf(b[11], b[12]), b[13]);
  const float v2 = fmaxf(fmaxf(b[14], b[15]), x);
  const float p = fmaxf(fmaxf(y, z), u), q = fmaxf(fmaxf(v, w), x2), r = fmaxf(fmaxf(y2, z2), u2);
  return fmaxf(fmaxf(fmaxf(p, q), r), v2);
}

// Largest of 16 values (chains of three-input maxima).
__device__ __forceinline__ float max16_8(const f32x16& a) {
  const float x = fmaxf(fmaxf(a[0], a[1]), a[2]), y = fmaxf(fmaxf(a[3], a[4]), a[5]);
  const float z = fmaxf(fmaxf(a[6], a[7]), a[8]), u = fmaxf(fmaxf(a[9], a[10]), a[11]);
  const float v = fmaxf(fmaxf(a[12], a[13]), a[14]);
  return fmaxf(fmaxf(fmaxf(x, y), z), fmaxf(fmaxf(u, v), a[15]));
}

// Packed tiles: S^T row m of a 32-key tile reads K row pi_slot8(m), so that
// lane half h holds in its registers r = 0..15 the keys 16 h + r of the tile:
// slot 2 t + h of tile t, key r of the slot.  P^T then packs into the B
// operand with lane half h's 32 bytes = slot h (tile 0) then slot 2 + h
// (tile 1), and a V^T row of the tile holds the slots' 16-byte chunks in the
// order 0, 2, 1, 3 (chunk c: slot 2 (c & 1) + (c >> 1)).
__device__ __forceinline__ int pi_slot8(int m) { return 16 * ((m >> 2) & 1) + 4 * (m >> 3) + (m & 3); }

// Four fp32 P values -> four E4M3 codes (P <= 2^8 < 448 needs no clamp).
__device__ __forceinline__ int pack_p(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  return __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
}

// One pipelined step n (as the bf16 stage): S^T(n+1) on the matrix cores
// with the softmax of block n and P(n-1) V(n-1); tile loads of V(n), K(n+3).
// c_cur / c_next: the logit multipliers of S^T tiles 0 and 1 of blocks n and
// n+1 for this lane (one per block, or per slot with packed tiles); the
// running max of block n+1 comes out scaled by them.  kr[h]: the K resource
// of the tile rows this wavefront's load instruction e covers, h = 64 e / D.
// The LDS pointers are restrict: a step reads other ring slots (v_lds) than
// it loads into (vl, kl), and saying so lets the compiler leave the loads in
// flight across the step's LDS reads.
template <int D, bool PARTIAL, bool SLOTS, typename MaskF>
__device__ __forceinline__ void step8(const i32x8 (&ka)[2][D / 64], const uint8_t* __restrict__ v_lds, int n,
                                      const i32x8& ones,
                                      const i32x8 (&qf)[D / 64], const f32x16 (&s_cur)[2], f32x16 (&s_next)[2],
                                      float& mx_next, const i32x8& p_prev, i32x8& p_cur, f32x16 (&o)[D / 32 + 1],
                                      const float (&c_cur)[SLOTS ? 2 : 1], const float (&c_next)[SLOTS ? 2 : 1],
                                      float mc, MaskF mask_next,
                                      int hf, __amdgpu_buffer_rsrc_t vr, uint8_t* __restrict__ vl,
                                      const uint32_t* voff, const __amdgpu_buffer_rsrc_t (&kr)[2],
                                      uint8_t* __restrict__ kl, const uint32_t* koff) {
  constexpr int DC = D / 64, DT = D / 32, NI = D / 32;
  s_next[0] = f32x16{};
#pragma unroll
  for (int c = 0; c < DC; ++c) s_next[0] = mfma8(ka[0][c], qf[c], s_next[0]);
  // V^T(n-1) operands after the first key tile's products (in the registers
  // its K operands held), and before this step's tile loads, so that no LDS
  // read of the step follows a direct-to-LDS load in program order (a read
  // the compiler cannot prove apart from one waits until it has landed).
  i32x8 va[DT];
  read_v8<D>(v_lds, hf, n, va);
  // Then the V tile's loads, the second key tile's products and the K tile's loads.
#pragma unroll
  for (int e = 0; e < NI; ++e)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(vr, (lds_ptr_t)(vl + e * 1024), 16, voff[e], 0, 0, 0);
  s_next[1] = f32x16{};
#pragma unroll
  for (int c = 0; c < DC; ++c) s_next[1] = mfma8(ka[1][c], qf[c], s_next[1]);
#pragma unroll
  for (int e = 0; e < NI; ++e)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(kr[(64 * e) / D], (lds_ptr_t)(kl + e * 1024), 16, koff[e], 0, 0, 0);
  int pw[8];
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      float p[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) p[e] = __builtin_amdgcn_exp2f(fmaf(s_cur[t][4 * r4 + e], c_cur[SLOTS ? t : 0], -mc));
      pw[4 * t + r4] = pack_p(p[0], p[1], p[2], p[3]);
    }
  p_cur = i32x8{pw[0], pw[1], pw[2], pw[3], pw[4], pw[5], pw[6], pw[7]};
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) o[dt] = mfma8(va[dt], p_prev, o[dt]);
  o[DT] = mfma8(ones, p_prev, o[DT]);
  // Packed tiles with a plan (SLOTS and PARTIAL): the caller masks S^T(n+1)
  // and takes its maximum after the step, and only masks tiles with a slot
  // of fewer than 16 keys.
  constexpr bool DEFER = SLOTS && PARTIAL;
  if (PARTIAL && !DEFER) mask_next(s_next);
  // (A multiplier is positive and rounding is monotone: the scaled maximum of
  // each tile is the maximum of its scaled values.)
  if constexpr (DEFER) (void)c_next;
  else if constexpr (SLOTS) mx_next = fmaxf(max16_8(s_next[0]) * c_next[0], max16_8(s_next[1]) * c_next[1]);
  else mx_next = max32(s_next[0], s_next[1]) * c_next[0];
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
// SLOTS: packed tiles, as in the bf16 packed stage: K codes in compact
// cube-major rows (k8 is then k8c), V codes in the slot layout
// [B, H, Nc, 4, D, 16] (v8 is v8s: each 16-key slot transposed), every tile
// four slot codes (cube, sub-slot, count).  With PARTIAL the tiles and the
// launch order come from the packing plan (plan, order); without it every
// tile is one whole cube of the list.  The logit multiplier and the key mask
// go per slot: lane half h holds slot 2 t + h of S^T tile t (pi_slot8).
template <int D, bool PARTIAL, bool RASTER, bool SLOTS>
__global__ void __launch_bounds__(kThreads8, 2) attn_fwd_fp8(const uint8_t* __restrict__ q8,
                                                              const float* __restrict__ qscale,
                                                              const uint8_t* __restrict__ k8,
                                                              const float* __restrict__ kscale,
                                                              const uint8_t* __restrict__ v8t,
                                                              const float* __restrict__ vscale,
                                                              const int32_t* __restrict__ idx,
                                                              const int32_t* __restrict__ plan,
                                                              const int32_t* __restrict__ order, int topk,
                                                              float scale_log2, uint16_t* __restrict__ oc,
                                                              float* __restrict__ lse, KGeom g, Placement pl) {
  constexpr bool PLAN = SLOTS && PARTIAL;
  constexpr int DC = D / 64, DT = D / 32, NI8 = D / 32;
  __shared__ __attribute__((aligned(16))) Smem8<D> sm;
  int i, h, b;
  if (!map_workgroup(g, pl, i, h, b)) return;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wq = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hf = lane >> 5, n = lane & 31;
  const long long bh = (long long)b * g.H + h;
  // PLAN: the query cubes of a head run in the order plan_order gives.
  if (PLAN) i = order[bh * g.nc + i];
  const uint8_t* kbase = k8 + bh * g.Np * D;
  const uint8_t* vbase = v8t + bh * g.Np * D;
  const float* ks = kscale + bh * g.nc;
  const int32_t* irow = idx + (bh * g.nc + i) * topk;
  const int32_t* prow_plan = PLAN ? plan + (bh * g.nc + i) * 4LL * (topk + 1) : nullptr;
  const int ntiles = PLAN ? prow_plan[0] : topk;
  const int q = 32 * wq + n;
  const auto blk = [&](int m) { return irow[m < ntiles ? m : ntiles - 1]; };
  // SLOTS: the code of slot s of tile m (tiles past the end: the last one).
  const auto slot = [&](int m, int sl) {
    const int mm = m < ntiles ? m : ntiles - 1;
    return PLAN ? prow_plan[4 * (mm + 1) + sl] : ((irow[mm] << 8) | (sl << 5) | 16);
  };
  // Per-block logit multiplier scale * log2(e) * sq_i * sk_j, kept above 0 so
  // that masked (-inf) logits stay -inf when a cube is all zero (scale 0).
  const float c_q = scale_log2 * qscale[bh * g.nc + i];
  const auto cblk = [&](int j) { return fmaxf(c_q * ks[j], 1e-30f); };
  // This lane's multipliers of S^T tiles 0 and 1 of tile m, and (SLOTS) its
  // slots' valid key counts.
  constexpr int NCT = SLOTS ? 2 : 1;  // multipliers (and slot counts) per lane and tile
  // full: every slot of the tile holds 16 valid keys (wave-uniform; PLAN only).
  const auto tile_c = [&](int m, float (&c)[NCT], int (&cnt)[NCT], bool& full) {
    full = true;
    if constexpr (SLOTS && !PLAN) {
      // Every tile is one whole cube: four full slots of the same cube.
      c[0] = c[1] = cblk(blk(m));
      cnt[0] = cnt[1] = 16;
    } else if constexpr (SLOTS) {
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int c0 = slot(m, 2 * t), c1 = slot(m, 2 * t + 1);
        // Both slots' key scales are loaded at their wave-uniform cubes and
        // only then picked per lane half: a lane-dependent index would make
        // the scale a vector load, and its wait would also cover every tile
        // load in flight.  The empty asm keeps the two loads apart.
        float s0 = ks[slot_cube(c0)], s1 = ks[slot_cube(c1)];
        asm volatile("" : "+v"(s0), "+v"(s1));
        c[t] = fmaxf(c_q * (hf ? s1 : s0), 1e-30f);
        cnt[t] = slot_count(hf ? c1 : c0);
        full = full & (slot_count(c0) == 16) & (slot_count(c1) == 16);
      }
    } else {
      c[0] = cblk(blk(m));
      cnt[0] = 64;
    }
  };
  const auto mask_of = [&](int m, const int (&cnt)[NCT]) {
    const int j = blk(m);
    return [=, &g](f32x16 (&sv)[2]) {
      if constexpr (SLOTS) {
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int r = 0; r < 16; ++r) sv[t][r] = r < cnt[t] ? sv[t][r] : -INFINITY;
      } else {
        mask_keys(sv[0], g, j, 0, hf);
        mask_keys(sv[1], g, j, 1, hf);
      }
    };
  };
  const Offsets8<D> off(wq, lane);
  // SLOTS: K tile rows of load instruction e lie in slot 2 wq + 64 e / D; the
  // resource of slot s is based so that the unchanged lane offsets of its
  // rows land on the slot's compact rows, with only its `count` rows in range.
  const auto k_rsrc = [&](int m, __amdgpu_buffer_rsrc_t (&r)[2]) {
    if constexpr (SLOTS) {
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int sg = 2 * wq + u, code = slot(m, sg), cnt = slot_count(code);
        const long long row0 = 64LL * slot_cube(code) + 16 * slot_sub(code) - 16 * sg;
        r[u] = make_rsrc(kbase + row0 * D, (m < ntiles && cnt) ? (unsigned)((16 * sg + cnt) * D) : 0u);
      }
    } else {
      r[0] = r[1] = make_rsrc(kbase + 64LL * blk(m) * D, m < ntiles ? 64 * D : 0u);
    }
  };
  // SLOTS: V^T tile instruction e of this lane fills row vr of the tile,
  // chunk v8_chunk(vr, lane % 4), which holds slot 2 (c & 1) + (c >> 1) of
  // chunk c; every lane reads its 16 bytes of that slot from the head's slot
  // layout.
  uint32_t vso[NI8];
  const __amdgpu_buffer_rsrc_t vhead = make_rsrc(vbase, (unsigned)(g.Np * D));
  const auto v_load = [&](int m) {
    if constexpr (SLOTS) {
      int sv[4];
#pragma unroll
      for (int sl = 0; sl < 4; ++sl) {
        const int code = slot(m, sl);
        sv[sl] = 4 * slot_cube(code) + slot_sub(code);
      }
#pragma unroll
      for (int e = 0; e < NI8; ++e) {
        const int vr = (wq * NI8 + e) * 16 + lane / 4, c = v8_chunk(vr, lane % 4);
        const int sx = (c & 1) ? ((c >> 1) ? sv[3] : sv[2]) : ((c >> 1) ? sv[1] : sv[0]);
        vso[e] = (uint32_t)((sx * D + vr) * 16);
      }
      return vhead;
    } else {
      return make_rsrc(vbase + 64LL * blk(m) * D, 64 * D);
    }
  };
  const uint32_t* voffs = SLOTS ? vso : off.v;
  __amdgpu_buffer_rsrc_t kr[2];

  {
    // V(-1) = 0, written before any tile load is in flight (an LDS store
    // after a direct-to-LDS load would wait for it to land).
    uint4* z = reinterpret_cast<uint4*>(sm.v[1]);
    for (int e = tid; e < D * 64 / 16; e += kThreads8) z[e] = make_uint4(0, 0, 0, 0);
  }
  k_rsrc(0, kr);
  issue8s<D>(kr, sm.k[0], wq, off.k);
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
  k_rsrc(1, kr);
  issue8s<D>(kr, sm.k[1], wq, off.k);
  k_rsrc(2, kr);
  issue8s<D>(kr, sm.k[2], wq, off.k);
  // Ones row of the normaliser: row 0 of an extra 32-row A operand.
  const int one = (n == 0) ? 0x38383838 : 0;  // four E4M3 ones
  const i32x8 ones = {one, one, one, one, one, one, one, one};
  f32x16 o[DT + 1];
#pragma unroll
  for (int dt = 0; dt <= DT; ++dt) o[dt] = f32x16{};
  float m_run = -INFINITY;  // running max, log2 units of the scaled logits
  const int prow = SLOTS ? pi_slot8(n) : pi_row(n);
  i32x8 p_prev = {};

  f32x16 s_cur[2];
  float c_cur[NCT];
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
    int cnt[NCT];
    bool full0;
    tile_c(0, c_cur, cnt, full0);
    if (PARTIAL) mask_of(0, cnt)(s_cur);
    if constexpr (SLOTS) mx_cur = fmaxf(max16_8(s_cur[0]) * c_cur[0], max16_8(s_cur[1]) * c_cur[1]);
    else mx_cur = max32(s_cur[0], s_cur[1]) * c_cur[0];
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
    float c_next[NCT];
    int cnt_next[NCT];
    bool full_next;
    tile_c(nb + 1, c_next, cnt_next, full_next);
    f32x16 s_next[2];
    float mx_next;
    i32x8 p_cur;
    const __amdgpu_buffer_rsrc_t vr = v_load(nb);
    // Past the last block the padding loads of K target a zero-size range: no memory traffic.
    k_rsrc(nb + 3, kr);
    step8<D, PARTIAL, SLOTS>(ka, sm.v[(u + 1) % 2], n, ones, qf, s_cur, s_next, mx_next, p_prev, p_cur, o, c_cur,
                             c_next, mc, mask_of(nb + 1, cnt_next), hf, vr, sm.v[u % 2] + wq * NI8 * 1024, voffs,
                             kr, sm.k[u % 3] + wq * NI8 * 1024, off.k);
    if constexpr (PLAN) {
      // Most tiles hold four full slots (16 valid keys each) and need no
      // mask; the test is on the tile's slot codes, so the branch is
      // wave-uniform.  The masking is the step's largest piece of vector work
      // after the exponentials.
      if (!full_next) mask_of(nb + 1, cnt_next)(s_next);
      mx_next = fmaxf(max16_8(s_next[0]) * c_next[0], max16_8(s_next[1]) * c_next[1]);
    }
    move = __builtin_amdgcn_ballot_w64(mx_next > m_run + kLazy8) != 0;
    if (resc) {
#pragma unroll
      for (int dt = 0; dt <= DT; ++dt) o[dt] *= alpha;
    }
    s_cur[0] = s_next[0];
    s_cur[1] = s_next[1];
#pragma unroll
    for (int t = 0; t < NCT; ++t) c_cur[t] = c_next[t];
    mx_cur = mx_next;
    p_prev = p_cur;
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
    wait_vmcnt<NI8>();
    pipeline_barrier();
    i32x8 va[DT];
    read_v8<D>(sm.v[(ntiles - 1) & 1], hf, n, va);
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

template <int D, bool PARTIAL, bool RASTER, bool SLOTS>
static void launch_fp8_t(const KGeom& g, const uint8_t* q8, const float* qs, const uint8_t* k8, const float* ks,
                         const uint8_t* v8, const float* vs, const int32_t* idx, const int32_t* plan,
                         const int32_t* order, int topk, float scale, uint16_t* oc, float* lse, hipStream_t s) {
  const Placement pl = make_placement(g);
  attn_fwd_fp8<D, PARTIAL, RASTER, SLOTS><<<dim3(grid_size(g)), dim3(kThreads8), 0, s>>>(
      q8, qs, k8, ks, v8, vs, idx, plan, order, topk, scale * 1.4426950408889634f, oc, lse, g, pl);
}

template <bool RASTER, bool SLOTS>
static void launch_fp8_any(const KGeom& g, const uint8_t* q8, const float* qs, const uint8_t* k8, const float* ks,
                           const uint8_t* v8, const float* vs, const int32_t* idx, const int32_t* plan,
                           const int32_t* order, int topk, float scale, uint16_t* oc, float* lse, hipStream_t s) {
#define VSA_FP8(DD, PP) \
  launch_fp8_t<DD, PP, RASTER, SLOTS>(g, q8, qs, k8, ks, v8, vs, idx, plan, order, topk, scale, oc, lse, s)
  if (g.D == 64) {
    if (g.partial) VSA_FP8(64, true);
    else VSA_FP8(64, false);
  } else {
    if (g.partial) VSA_FP8(128, true);
    else VSA_FP8(128, false);
  }
#undef VSA_FP8
}

hipError_t launch_attn_fwd_fp8(const KGeom& g, const uint8_t* q8, const float* qs, const uint8_t* k8,
                               const float* ks, const uint8_t* v8t, const float* vs, const int32_t* idx, int topk,
                               float scale, bool raster_out, uint16_t* o, float* lse, hipStream_t s) {
  if (raster_out)
    launch_fp8_any<true, false>(g, q8, qs, k8, ks, v8t, vs, idx, nullptr, nullptr, topk, scale, o, lse, s);
  else launch_fp8_any<false, false>(g, q8, qs, k8, ks, v8t, vs, idx, nullptr, nullptr, topk, scale, o, lse, s);
  return hipGetLastError();
}

hipError_t launch_attn_fwd_fp8_packed(const KGeom& g, const uint8_t* q8, const float* qs, const uint8_t* k8c,
                                      const float* ks, const uint8_t* v8s, const float* vs, const int32_t* idx,
                                      int topk, float scale, bool raster_out, uint16_t* o, float* lse, void* ws,
                                      hipStream_t s) {
  const int32_t* plan = nullptr;
  const int32_t* order = nullptr;
  if (g.partial) {
    const hipError_t e = launch_packed_plan(g, idx, topk, ws, s);
    if (e != hipSuccess) return e;
    plan = static_cast<const int32_t*>(ws);
    order = plan + (long long)g.B * g.H * g.nc * 4LL * (topk + 1);
  }
  if (raster_out) launch_fp8_any<true, true>(g, q8, qs, k8c, ks, v8s, vs, idx, plan, order, topk, scale, o, lse, s);
  else launch_fp8_any<false, true>(g, q8, qs, k8c, ks, v8s, vs, idx, plan, order, topk, scale, o, lse, s);
  return hipGetLastError();
}

}  // namespace vsa
