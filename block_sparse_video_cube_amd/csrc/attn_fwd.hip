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
//    (buffer_load_dwordx4 ... lds) through per-tile buffer resources,
//    double-buffered: the loads of block n+1 are in flight while block n is
//    computed.  Each 16-byte chunk is placed with an
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

#include "common.h"

namespace vsa {

namespace {

constexpr int kThreads = 256;
constexpr float kLazyLog2 = 8.f;

// Wait until every global load of this wavefront has completed, including the
// direct-to-LDS tile loads (s_waitcnt vmcnt(0); gfx9 encoding, other
// counters left at their maximum).  The workgroup fence of __syncthreads()
// treats those loads as loads and does not wait for them by itself.
__device__ __forceinline__ void wait_tile_loads() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Key row loaded by A-operand lane row m (0..31) of a 32-key tile.  With it,
// accumulator register r of lane half hf holds key 16*(r/8) + 8*hf + r%8.
__device__ __forceinline__ int pi_row(int m) {
  const int gq = m >> 3, hq = (m >> 2) & 1, rr = m & 3;
  return 16 * (gq >> 1) + 8 * hq + 4 * (gq & 1) + rr;
}

// 16-byte chunk swizzles.
template <int D>
__device__ __forceinline__ int k_swz(int row) {
  return (D == 128) ? (row & 15) : ((row >> 1) & 7);
}
__device__ __forceinline__ int v_swz(int row) { return (row >> 1) & 7; }

template <int D>
struct Smem {
  uint16_t k[2][64 * D];
  uint16_t v[2][D * 64];
};

// Per-lane byte offsets of this wave's share of one K tile and one V^T tile.
// Every buffer_load_dwordx4 ... lds writes 64 consecutive 16-byte LDS slots;
// lane L fills slot L with the global chunk that the swizzle maps there.
template <int D>
struct TileOffsets {
  static constexpr int KRPI = 512 / D;  // K rows per 1 KB instruction
  static constexpr int NI = D / 32;     // instructions per wave per tile
  uint32_t k[NI], v[NI];
  __device__ __forceinline__ TileOffsets(int w, int lane) {
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int row = (w * NI + i) * KRPI + lane / (D / 8);
      k[i] = (uint32_t)(row * D + ((lane % (D / 8)) ^ k_swz<D>(row)) * 8) * 2u;
      const int vrow = (w * NI + i) * 8 + (lane >> 3);
      v[i] = (uint32_t)(vrow * 64 + ((lane & 7) ^ v_swz(vrow)) * 8) * 2u;
    }
  }
};

// Issue the direct-to-LDS loads of one K tile and one V^T tile (this wave's
// share).  The buffer resources cover exactly one tile each, so every load is
// range-checked by the hardware.
template <int D>
__device__ __forceinline__ void load_tiles(const uint16_t* ktile, const uint16_t* vtile, uint16_t* klds,
                                           uint16_t* vlds, int w, const TileOffsets<D>& off) {
  constexpr int KRPI = TileOffsets<D>::KRPI, NI = TileOffsets<D>::NI;
  const __amdgpu_buffer_rsrc_t kr = make_rsrc(ktile, 64 * D * 2);
  const __amdgpu_buffer_rsrc_t vr = make_rsrc(vtile, 64 * D * 2);
#pragma unroll
  for (int i = 0; i < NI; ++i)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(kr, (lds_ptr_t)(klds + (w * NI + i) * KRPI * D), 16, off.k[i], 0, 0, 0);
#pragma unroll
  for (int i = 0; i < NI; ++i)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(vr, (lds_ptr_t)(vlds + (w * NI + i) * 8 * 64), 16, off.v[i], 0, 0, 0);
}

template <int D>
__device__ __forceinline__ void block_step(const uint16_t* klds, const uint16_t* vlds, const bf16x8 (&qf)[D / 16],
                                           f32x16 (&o)[D / 32], float& m_run, float& l_run, bool partial,
                                           const KGeom& g, int j, int wk, int hf, int n, int prow,
                                           float scale_log2, float lazy_raw) {
  constexpr int DC = D / 16, DT = D / 32;
  // S^T (32 keys x 32 queries) for this wave's key half: all K fragments
  // first, then the MFMA chain.
  const int krow = 32 * wk + prow;
  bf16x8 ka[DC];
#pragma unroll
  for (int dc = 0; dc < DC; ++dc)
    ka[dc] = *reinterpret_cast<const bf16x8*>(klds + krow * D + (((2 * dc + hf) ^ k_swz<D>(krow)) * 8));
  f32x16 s = f32x16{};
#pragma unroll
  for (int dc = 0; dc < DC; ++dc) s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[dc], qf[dc], s, 0, 0, 0);
  // V^T fragments for this block, read while the softmax runs.
  bf16x8 va[DT][2];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) {
    const int vrow = 32 * dt + n;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const int chunk = 4 * wk + 2 * kk + hf;
      va[dt][kk] = *reinterpret_cast<const bf16x8*>(vlds + vrow * 64 + ((chunk ^ v_swz(vrow)) * 8));
    }
  }
  if (partial) {
    int ct, cy, cx;
    cube_coords(g, j, ct, cy, cx);
    if (!cube_full(g, ct, cy, cx)) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = 32 * wk + 16 * (r >> 3) + 8 * hf + (r & 7);
        if (!local_valid(g, ct, cy, cx, key)) s[r] = -INFINITY;
      }
    }
  }
  // Max over this lane's 16 keys.  The reference max moves only when the
  // block exceeds it by more than kLazyLog2 (log2 units); since each lane
  // half's max bounds the row max from below, the rare move is decided per
  // half and only then is the row max taken across lane ^ 32.  A half that
  // holds padded keys only (mx = -inf) never triggers a move.
  float mx = fmaxf(s[0], s[1]);
#pragma unroll
  for (int r = 2; r < 16; ++r) mx = fmaxf(mx, s[r]);
  if (__builtin_amdgcn_ballot_w64(mx > m_run + lazy_raw)) {
    const float row_max = fmaxf(mx, __shfl_xor(mx, 32));
    const bool grow = row_max > m_run + lazy_raw;
    const float alpha = grow ? __builtin_amdgcn_exp2f((m_run - row_max) * scale_log2) : 1.f;
    m_run = grow ? row_max : m_run;
    l_run *= alpha;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) o[dt] *= alpha;
  }
  // Until a valid key has been seen every logit is -inf and p must be 0.
  const float mc = (m_run == -INFINITY) ? 0.f : m_run * scale_log2;
  // P rounded once to bf16 (v_cvt_pk_bf16_f32); the normaliser sums the same
  // rounded values (v_dot2_f32_bf16 against 1.0), so the weights applied to V
  // sum exactly to the normaliser.
  uint32_t pw[8];
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    const float p0 = __builtin_amdgcn_exp2f(fmaf(s[2 * r], scale_log2, -mc));
    const float p1 = __builtin_amdgcn_exp2f(fmaf(s[2 * r + 1], scale_log2, -mc));
    const bf16x2 pk = __builtin_convertvector((f32x2){p0, p1}, bf16x2);
    l_run = __builtin_amdgcn_fdot2_f32_bf16(pk, ones, l_run, false);
    pw[r] = __builtin_bit_cast(uint32_t, pk);
  }
  bf16x8 pb[2];
  pb[0] = __builtin_bit_cast(bf16x8, make_uint4(pw[0], pw[1], pw[2], pw[3]));
  pb[1] = __builtin_bit_cast(bf16x8, make_uint4(pw[4], pw[5], pw[6], pw[7]));
  // O^T += V^T P^T over this wave's 32 keys (2 chunks of 16).
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[dt][kk], pb[kk], o[dt], 0, 0, 0);
}

template <int D>
__global__ void __launch_bounds__(kThreads, 2) attn_fwd(const uint16_t* __restrict__ qc,
                                                        const uint16_t* __restrict__ kc,
                                                        const uint16_t* __restrict__ vt,
                                                        const int32_t* __restrict__ idx, int topk, float scale,
                                                        float scale_log2, uint16_t* __restrict__ oc,
                                                        float* __restrict__ oc_f32, float* __restrict__ lse,
                                                        KGeom g) {
  constexpr int DC = D / 16, DT = D / 32;
  __shared__ __attribute__((aligned(16))) Smem<D> sm;

  const int i = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wq = w & 1, wk = w >> 1;  // wave-uniform
  const int hf = lane >> 5, n = lane & 31;
  const long long bh = (long long)b * g.H + h;
  const uint16_t* kbase = kc + bh * g.Np * D;
  const uint16_t* vbase = vt + bh * g.Np * D;
  const int32_t* irow = idx + (bh * g.nc + i) * topk;
  const int q = 32 * wq + n;

  // First tiles in flight before anything else.
  const TileOffsets<D> toff(w, lane);
  {
    const int j0 = irow[0];
    load_tiles<D>(kbase + 64LL * j0 * D, vbase + 64LL * j0 * D, sm.k[0], sm.v[0], w, toff);
  }

  bf16x8 qf[DC];
  {
    const uint16_t* qrow = qc + (bh * g.Np + 64LL * i + q) * D;
#pragma unroll
    for (int dc = 0; dc < DC; ++dc) qf[dc] = *reinterpret_cast<const bf16x8*>(qrow + 16 * dc + 8 * hf);
  }
  f32x16 o[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) o[dt] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;
  const int prow = pi_row(n);
  const float lazy_raw = kLazyLog2 / scale_log2;

  // Two blocks per trip so that both LDS buffers are compile-time distinct.
  for (int jb = 0; jb < topk; jb += 2) {
    {
      const int j = irow[jb];
      wait_tile_loads();
      __syncthreads();  // tiles of block jb have landed (every wave waited for its own loads)
      if (jb + 1 < topk) {
        const int jn = irow[jb + 1];
        load_tiles<D>(kbase + 64LL * jn * D, vbase + 64LL * jn * D, sm.k[1], sm.v[1], w, toff);
      }
      block_step<D>(sm.k[0], sm.v[0], qf, o, m_run, l_run, g.partial, g, j, wk, hf, n, prow, scale_log2,
                    lazy_raw);
    }
    if (jb + 1 < topk) {
      const int j = irow[jb + 1];
      wait_tile_loads();
      __syncthreads();
      if (jb + 2 < topk) {
        const int jn = irow[jb + 2];
        load_tiles<D>(kbase + 64LL * jn * D, vbase + 64LL * jn * D, sm.k[0], sm.v[0], w, toff);
      }
      block_step<D>(sm.k[1], sm.v[1], qf, o, m_run, l_run, g.partial, g, j, wk, hf, n, prow, scale_log2,
                    lazy_raw);
    }
  }

  // Merge the two key halves: wavefronts with wk = 1 hand (m, l, O^T) over.
  l_run += __shfl_xor(l_run, 32);
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
        v[e] = o[dt][r] * c0 + xo[(dt * 16 + r) * 64 + lane] * c1;
      }
      *reinterpret_cast<uint2*>(orow + d) = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
      if (oc_f32) *reinterpret_cast<float4*>(oc_f32 + row * D + d) = make_float4(v[0], v[1], v[2], v[3]);
    }
  if (lse && hf == 0) lse[row] = m * scale + logf(l_tot);
}

}  // namespace

hipError_t launch_attn_fwd(const KGeom& g, const uint16_t* qc, const uint16_t* kc, const uint16_t* vt,
                           const int32_t* idx, int topk, float scale, uint16_t* oc, float* oc_f32, float* lse,
                           hipStream_t s) {
  const dim3 grid(g.nc, g.H, g.B);
  const float scale_log2 = scale * 1.4426950408889634f;
  if (g.D == 64)
    hipLaunchKernelGGL(attn_fwd<64>, grid, dim3(kThreads), 0, s, qc, kc, vt, idx, topk, scale, scale_log2, oc,
                       oc_f32, lse, g);
  else
    hipLaunchKernelGGL(attn_fwd<128>, grid, dim3(kThreads), 0, s, qc, kc, vt, idx, topk, scale, scale_log2, oc,
                       oc_f32, lse, g);
  return hipGetLastError();
}

}  // namespace vsa
