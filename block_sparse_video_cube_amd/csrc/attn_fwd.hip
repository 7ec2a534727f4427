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
// gfx950 mapping.  One workgroup = one query cube = 2 wavefronts x 32 query
// rows.  Per selected key cube the K tile (64 x D, token-major) and the V tile
// (D x 64, stored transposed) are staged in LDS with an XOR swizzle of their
// 16-byte chunks.  Each wavefront computes the transposed score tile
// S^T = K Q^T with v_mfma_f32_32x32x16_bf16, so that a lane owns one query
// column: row max and row sum are in-lane plus one exchange with lane ^ 32.
// The A-operand rows of K are loaded in the order pi (below), which makes the
// accumulator of S^T already the B operand layout of O^T = V^T P^T: P never
// leaves registers.  O^T accumulates in fp32 and a lane's rescale factor is a
// per-lane scalar.
#include <math.h>

#include "common.h"

namespace vsa {

namespace {

constexpr int kWaves = 2;
constexpr int kThreads = 64 * kWaves;

// Key row loaded by A-operand lane row m (0..31) of a 32-key tile.  With it,
// accumulator register r of lane half hf holds key 16*(r/8) + 8*hf + r%8.
__device__ __forceinline__ int pi_row(int m) {
  const int gq = m >> 3, hq = (m >> 2) & 1, rr = m & 3;
  return 16 * (gq >> 1) + 8 * hq + 4 * (gq & 1) + rr;
}

// 16-byte chunk swizzles (conflict-free A-operand reads, see header comment).
template <int D>
__device__ __forceinline__ int k_swz(int row) {
  return (D == 128) ? (row & 15) : ((row >> 1) & 7);
}
__device__ __forceinline__ int v_swz(int row) { return (row >> 1) & 7; }

template <int D>
__global__ void __launch_bounds__(kThreads) attn_fwd(const uint16_t* __restrict__ qc,
                                                     const uint16_t* __restrict__ kc,
                                                     const uint16_t* __restrict__ vt,
                                                     const int32_t* __restrict__ idx, int topk,
                                                     float scale, float scale_log2, uint16_t* __restrict__ oc,
                                                     float* __restrict__ oc_f32, float* __restrict__ lse,
                                                     KGeom g) {
  constexpr int DC = D / 16;  // 16-wide d chunks of S^T
  constexpr int DT = D / 32;  // 32-wide d tiles of O^T
  constexpr int CH = D / 8;   // 16-byte chunks per K row
  __shared__ __attribute__((aligned(16))) uint16_t k_lds[64 * D];
  __shared__ __attribute__((aligned(16))) uint16_t v_lds[D * 64];

  const int i = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int hf = lane >> 5, n = lane & 31;
  const long long bh = (long long)b * g.H + h;
  const uint16_t* kbase = kc + bh * g.Np * D;
  const uint16_t* vbase = vt + bh * g.Np * D;
  const int32_t* irow = idx + (bh * g.nc + i) * topk;
  const int q = 32 * w + n;  // query row of this lane within the cube

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

  for (int jb = 0; jb < topk; ++jb) {
    const int j = irow[jb];
    __syncthreads();  // everybody is done with the previous tiles
    {
      const uint4* ksrc = reinterpret_cast<const uint4*>(kbase + 64LL * j * D);
#pragma unroll
      for (int f = tid; f < 64 * CH; f += kThreads) {
        const int row = f / CH, ch = f % CH;
        *reinterpret_cast<uint4*>(k_lds + row * D + ((ch ^ k_swz<D>(row)) * 8)) = ksrc[f];
      }
      const uint4* vsrc = reinterpret_cast<const uint4*>(vbase + 64LL * j * D);
#pragma unroll
      for (int f = tid; f < D * 8; f += kThreads) {
        const int row = f >> 3, ch = f & 7;
        *reinterpret_cast<uint4*>(v_lds + row * 64 + ((ch ^ v_swz(row)) * 8)) = vsrc[f];
      }
    }
    __syncthreads();

    // S^T = K Q^T for keys 0..31 (mt = 0) and 32..63 (mt = 1).
    f32x16 s[2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      s[mt] = f32x16{};
      const int krow = 32 * mt + prow;
#pragma unroll
      for (int dc = 0; dc < DC; ++dc) {
        const bf16x8 a =
            *reinterpret_cast<const bf16x8*>(k_lds + krow * D + (((2 * dc + hf) ^ k_swz<D>(krow)) * 8));
        s[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[dc], s[mt], 0, 0, 0);
      }
    }

    // Padded keys of a partial cube take no weight.
    int ct, cy, cx;
    cube_coords(g, j, ct, cy, cx);
    if (!cube_full(g, ct, cy, cx)) {
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = 32 * mt + 16 * (r >> 3) + 8 * hf + (r & 7);
          if (!local_valid(g, ct, cy, cx, key)) s[mt][r] = -INFINITY;
        }
    }

    // Online softmax for query column n: lane half hf holds 32 of its 64 keys.
    float mx = s[0][0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s[0][r]);
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[1][r]);
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx);
    const float alpha = __builtin_amdgcn_exp2f((m_run - m_new) * scale_log2);
    const float mc = m_new * scale_log2;
    m_run = m_new;

    bf16x8 pb[4];
    float psum = 0.f;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = __builtin_amdgcn_exp2f(fmaf(s[mt][r], scale_log2, -mc));
        psum += p;
        pb[2 * mt + (r >> 3)][r & 7] = __builtin_bit_cast(__bf16, f32_to_bf16(p));
      }
    l_run = l_run * alpha + psum;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) o[dt] *= alpha;

    // O^T += V^T P^T over 4 chunks of 16 keys.
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const int vrow = 32 * dt + n;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const bf16x8 a =
            *reinterpret_cast<const bf16x8*>(v_lds + vrow * 64 + (((2 * kk + hf) ^ v_swz(vrow)) * 8));
        o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[kk], o[dt], 0, 0, 0);
      }
    }
  }

  // Epilogue: normalise, round once to bf16, store.
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const float inv = 1.f / l_tot;
  const long long row = bh * g.Np + 64LL * i + q;
  uint16_t* orow = oc + row * D;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int gq = 0; gq < 4; ++gq) {
      const int d = 32 * dt + 8 * gq + 4 * hf;
      const float v0 = o[dt][4 * gq + 0] * inv, v1 = o[dt][4 * gq + 1] * inv;
      const float v2 = o[dt][4 * gq + 2] * inv, v3 = o[dt][4 * gq + 3] * inv;
      *reinterpret_cast<uint2*>(orow + d) = make_uint2(pack_bf16x2(v0, v1), pack_bf16x2(v2, v3));
      if (oc_f32) *reinterpret_cast<float4*>(oc_f32 + row * D + d) = make_float4(v0, v1, v2, v3);
    }
  if (lse && hf == 0) lse[row] = m_run * scale + logf(l_tot);
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
