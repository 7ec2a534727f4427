// Linear-attention branch over the unselected cubes, and the combine.
//
// Pairing the block-sparse branch with a low-rank linear branch keeps global
// context when 97 % of the blocks are skipped (SparkDiffusion article,
// paragraph 3, RoLA); a trainable sparse + linear attention brings attention
// cost down to linear (TurboDiffusion article, section
// "稀疏、蒸馏与全链路量化", SLA).  Convention: phi(x) = elu(x) + 1 and, for
// query cube i with unselected cubes U,
//   O_lin = phi(Q) (sum_U phi(K)^T V) / (phi(Q) . sum_U phi(K)),  0 if U empty,
// and the layer output is O_sparse + O_lin, rounded once to bf16.
//
// Instead of one D x D state per cube, the unselected sum is the total minus
// the selected part, and the selected part is taken block by block exactly
// as the fine stage does, with phi weights in place of the softmax:
//   num = phi(Q) S_tot - sum_{j in sel} (phi(Q) phi(K_j)^T) V_j
//   den = phi(Q) z_tot - sum_{j in sel} rowsum(phi(Q) phi(K_j)^T).
//
// Kernels:
//   lin_state   per (b, h, group of 8 cubes): phi(K) (bf16, padded rows 0)
//               written token-major for lin_apply, and partial
//               S = phi(K)^T V (bf16 MFMA, fp32 accumulate) and z = sum phi(K);
//   lin_reduce  per (b, h): S_tot^T split into bf16 hi + lo halves, z_tot;
//   lin_apply   per (b, h, query cube): num / den and the combine.
#include <math.h>

#include "common.h"

namespace vsa {

namespace {

constexpr int kGroup = 8;  // cubes per partial state

__device__ __forceinline__ float phi(float x) { return x > 0.f ? x + 1.f : __expf(x); }

__device__ __forceinline__ int pi_row(int m) {
  const int gq = m >> 3, hq = (m >> 2) & 1, rr = m & 3;
  return 16 * (gq >> 1) + 8 * hq + 4 * (gq & 1) + rr;
}
template <int D>
__device__ __forceinline__ int k_swz(int row) {
  return (D == 128) ? (row & 15) : ((row >> 1) & 7);
}
__device__ __forceinline__ int v_swz(int row) { return (row >> 1) & 7; }

struct LinWs {
  uint16_t* fk;     // [B, H, Np, D] bf16 phi(K), token-major
  float* s_part;    // [B, H, G, D, D]
  float* z_part;    // [B, H, G, D]
  uint16_t* st_hi;  // [B, H, D(e), D(d)] bf16
  uint16_t* st_lo;  // [B, H, D(e), D(d)] bf16
  float* z_tot;     // [B, H, D]
};

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

LinWs carve(const KGeom& g, void* ws, size_t* total) {
  const size_t bh = (size_t)g.B * g.H;
  const size_t G = (g.nc + kGroup - 1) / kGroup;
  const size_t D = g.D;
  size_t off = 0;
  char* base = static_cast<char*>(ws);
  LinWs w;
  w.fk = reinterpret_cast<uint16_t*>(base + off);
  off += align256(bh * g.Np * D * 2);
  w.s_part = reinterpret_cast<float*>(base + off);
  off += align256(bh * G * D * D * 4);
  w.z_part = reinterpret_cast<float*>(base + off);
  off += align256(bh * G * D * 4);
  w.st_hi = reinterpret_cast<uint16_t*>(base + off);
  off += align256(bh * D * D * 2);
  w.st_lo = reinterpret_cast<uint16_t*>(base + off);
  off += align256(bh * D * D * 2);
  w.z_tot = reinterpret_cast<float*>(base + off);
  off += align256(bh * D * 4);
  if (total) *total = off;
  return w;
}

template <int D>
__global__ void __launch_bounds__(256) lin_state(const uint16_t* __restrict__ kc, const uint16_t* __restrict__ vt,
                                                 LinWs ws, KGeom g) {
  constexpr int CH = D / 8;
  constexpr int RGS = 256 / CH;                 // threads sharing one d chunk
  constexpr int NT = (D == 128) ? 4 : 1;        // e tiles per wave
  __shared__ __attribute__((aligned(16))) uint16_t fkT[D * 64];
  __shared__ float zred[RGS][D];
  const int grp = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, hf = lane >> 5, n = lane & 31;
  const long long bh = (long long)b * g.H + h;
  const int G = (g.nc + kGroup - 1) / kGroup;
  const int mt = (D == 128) ? w : (w >> 1);
  const int nt0 = (D == 128) ? 0 : (w & 1);
  f32x16 acc[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) acc[t] = f32x16{};
  float zacc[8] = {};
  const int ch = tid % CH;

  for (int c = grp * kGroup; c < min(g.nc, (grp + 1) * kGroup); ++c) {
    int ct, cy, cx;
    cube_coords(g, c, ct, cy, cx);
    __syncthreads();
    const uint4* ksrc = reinterpret_cast<const uint4*>(kc + (bh * g.Np + 64LL * c) * D);
    uint4* fdst = reinterpret_cast<uint4*>(ws.fk + (bh * g.Np + 64LL * c) * D);
    for (int f = tid; f < 64 * CH; f += 256) {
      const int row = f / CH;
      const bool valid = local_valid(g, ct, cy, cx, row);
      const uint4 raw = ksrc[f];
      const uint32_t wv[4] = {raw.x, raw.y, raw.z, raw.w};
      uint32_t outw[4];
#pragma unroll
      for (int e2 = 0; e2 < 4; ++e2) {
        const float x0 = __uint_as_float(wv[e2] << 16), x1 = __uint_as_float(wv[e2] & 0xFFFF0000u);
        const uint16_t p0 = valid ? f32_to_bf16(phi(x0)) : 0, p1 = valid ? f32_to_bf16(phi(x1)) : 0;
        zacc[2 * e2] += bf16_to_f32(p0);
        zacc[2 * e2 + 1] += bf16_to_f32(p1);
        outw[e2] = (uint32_t)p0 | ((uint32_t)p1 << 16);
        const int d0 = 8 * ch + 2 * e2;
        fkT[d0 * 64 + (((row >> 3) ^ v_swz(d0)) * 8) + (row & 7)] = p0;
        fkT[(d0 + 1) * 64 + (((row >> 3) ^ v_swz(d0 + 1)) * 8) + (row & 7)] = p1;
      }
      fdst[f] = make_uint4(outw[0], outw[1], outw[2], outw[3]);
    }
    __syncthreads();
    const uint16_t* vcube = vt + (bh * g.Np + 64LL * c) * D;
    const int drow = 32 * mt + n;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(fkT + drow * 64 + (((2 * kk + hf) ^ v_swz(drow)) * 8));
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const int e = 32 * (nt0 + t) + n;
        const bf16x8 bv = *reinterpret_cast<const bf16x8*>(vcube + e * 64 + 16 * kk + 8 * hf);
        acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bv, acc[t], 0, 0, 0);
      }
    }
  }
  // Partial state out: S[d][e], d = 32 mt + 8 (r/4) + 4 hf + r%4, e = 32 nt + n.
  float* sp = ws.s_part + (bh * G + grp) * (long long)D * D;
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int d = 32 * mt + 8 * (r >> 2) + 4 * hf + (r & 3);
      const int e = 32 * (nt0 + t) + n;
      sp[d * D + e] = acc[t][r];
    }
#pragma unroll
  for (int e = 0; e < 8; ++e) zred[tid / CH][8 * ch + e] = zacc[e];
  __syncthreads();
  if (tid < D) {
    float s = 0.f;
    for (int r = 0; r < RGS; ++r) s += zred[r][tid];
    ws.z_part[(bh * G + grp) * D + tid] = s;
  }
}

template <int D>
__global__ void __launch_bounds__(256) lin_reduce(LinWs ws, KGeom g) {
  const long long bh = blockIdx.x;
  const int G = (g.nc + kGroup - 1) / kGroup;
  const float* sp = ws.s_part + bh * G * (long long)D * D;
  for (int f = threadIdx.x; f < D * D; f += 256) {
    const int d = f / D, e = f % D;
    float s = 0.f;
    for (int gi = 0; gi < G; ++gi) s += sp[(long long)gi * D * D + f];
    const uint16_t hi = f32_to_bf16(s);
    const uint16_t lo = f32_to_bf16(s - bf16_to_f32(hi));
    ws.st_hi[bh * D * D + e * D + d] = hi;
    ws.st_lo[bh * D * D + e * D + d] = lo;
  }
  if (threadIdx.x < D) {
    float s = 0.f;
    for (int gi = 0; gi < G; ++gi) s += ws.z_part[(bh * G + gi) * D + threadIdx.x];
    ws.z_tot[bh * D + threadIdx.x] = s;
  }
}

template <int D>
__global__ void __launch_bounds__(128) lin_apply(const uint16_t* __restrict__ qc, const uint16_t* __restrict__ vt,
                                                 const int32_t* __restrict__ idx, int topk,
                                                 const float* __restrict__ o_sparse, uint16_t* __restrict__ oc,
                                                 LinWs ws, KGeom g) {
  constexpr int DC = D / 16, DT = D / 32, CH = D / 8;
  __shared__ __attribute__((aligned(16))) uint16_t f_lds[64 * D];
  __shared__ __attribute__((aligned(16))) uint16_t v_lds[D * 64];
  const int i = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, hf = lane >> 5, n = lane & 31;
  const long long bh = (long long)b * g.H + h;
  const int q = 32 * w + n;
  const long long row = bh * g.Np + 64LL * i + q;
  const bool empty_u = topk >= g.nc;

  // phi(Q) fragments (bf16) and phi(Q) . z_tot.
  bf16x8 fq[DC];
  float den_part = 0.f;
  {
    const uint16_t* qrow = qc + row * D;
    const float* zt = ws.z_tot + bh * D;
#pragma unroll
    for (int dc = 0; dc < DC; ++dc) {
      const uint4 raw = *reinterpret_cast<const uint4*>(qrow + 16 * dc + 8 * hf);
      const uint32_t wv[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
      for (int e2 = 0; e2 < 4; ++e2) {
        const uint16_t p0 = f32_to_bf16(phi(__uint_as_float(wv[e2] << 16)));
        const uint16_t p1 = f32_to_bf16(phi(__uint_as_float(wv[e2] & 0xFFFF0000u)));
        fq[dc][2 * e2] = __builtin_bit_cast(__bf16, p0);
        fq[dc][2 * e2 + 1] = __builtin_bit_cast(__bf16, p1);
        const int d = 16 * dc + 8 * hf + 2 * e2;
        den_part += bf16_to_f32(p0) * zt[d] + bf16_to_f32(p1) * zt[d + 1];
      }
    }
  }
  // num^T = S_tot^T phi(Q)^T (hi + lo halves).
  f32x16 num[DT], corr[DT];
  const uint16_t* sth = ws.st_hi + bh * D * D;
  const uint16_t* stl = ws.st_lo + bh * D * D;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) {
    num[dt] = f32x16{};
    corr[dt] = f32x16{};
    const int e = 32 * dt + n;
#pragma unroll
    for (int dc = 0; dc < DC; ++dc) {
      const bf16x8 ah = *reinterpret_cast<const bf16x8*>(sth + e * D + 16 * dc + 8 * hf);
      const bf16x8 al = *reinterpret_cast<const bf16x8*>(stl + e * D + 16 * dc + 8 * hf);
      num[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah, fq[dc], num[dt], 0, 0, 0);
      num[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al, fq[dc], num[dt], 0, 0, 0);
    }
  }

  // Selected part, block by block.
  float dcorr = 0.f;
  const int32_t* irow = idx + (bh * g.nc + i) * topk;
  const uint16_t* fkb = ws.fk + bh * g.Np * D;
  const uint16_t* vb = vt + bh * g.Np * D;
  const int prow = pi_row(n);
  for (int jb = 0; jb < (empty_u ? 0 : topk); ++jb) {
    const int j = irow[jb];
    __syncthreads();
    const uint4* fsrc = reinterpret_cast<const uint4*>(fkb + 64LL * j * D);
    for (int f = tid; f < 64 * CH; f += 128) {
      const int r = f / CH, ch = f % CH;
      *reinterpret_cast<uint4*>(f_lds + r * D + ((ch ^ k_swz<D>(r)) * 8)) = fsrc[f];
    }
    const uint4* vsrc = reinterpret_cast<const uint4*>(vb + 64LL * j * D);
    for (int f = tid; f < D * 8; f += 128) {
      const int r = f >> 3, ch = f & 7;
      *reinterpret_cast<uint4*>(v_lds + r * 64 + ((ch ^ v_swz(r)) * 8)) = vsrc[f];
    }
    __syncthreads();
    bf16x8 pb[4];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      f32x16 s = f32x16{};
      const int krow = 32 * mt + prow;
#pragma unroll
      for (int dc = 0; dc < DC; ++dc) {
        const bf16x8 a =
            *reinterpret_cast<const bf16x8*>(f_lds + krow * D + (((2 * dc + hf) ^ k_swz<D>(krow)) * 8));
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, fq[dc], s, 0, 0, 0);
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const uint16_t pbits = f32_to_bf16(s[r]);
        dcorr += bf16_to_f32(pbits);
        pb[2 * mt + (r >> 3)][r & 7] = __builtin_bit_cast(__bf16, pbits);
      }
    }
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const int vrow = 32 * dt + n;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const bf16x8 a =
            *reinterpret_cast<const bf16x8*>(v_lds + vrow * 64 + (((2 * kk + hf) ^ v_swz(vrow)) * 8));
        corr[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[kk], corr[dt], 0, 0, 0);
      }
    }
  }
  const float den = (den_part + __shfl_xor(den_part, 32)) - (dcorr + __shfl_xor(dcorr, 32));
  const float inv = empty_u ? 0.f : 1.f / den;
  const float* osrc = o_sparse + row * D;
  uint16_t* odst = oc + row * D;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int gq = 0; gq < 4; ++gq) {
      const int e = 32 * dt + 8 * gq + 4 * hf;
      const float4 os = *reinterpret_cast<const float4*>(osrc + e);
      const float l0 = empty_u ? 0.f : (num[dt][4 * gq + 0] - corr[dt][4 * gq + 0]) * inv;
      const float l1 = empty_u ? 0.f : (num[dt][4 * gq + 1] - corr[dt][4 * gq + 1]) * inv;
      const float l2 = empty_u ? 0.f : (num[dt][4 * gq + 2] - corr[dt][4 * gq + 2]) * inv;
      const float l3 = empty_u ? 0.f : (num[dt][4 * gq + 3] - corr[dt][4 * gq + 3]) * inv;
      *reinterpret_cast<uint2*>(odst + e) =
          make_uint2(pack_bf16x2(os.x + l0, os.y + l1), pack_bf16x2(os.z + l2, os.w + l3));
    }
}

}  // namespace

size_t linear_workspace_bytes(const KGeom& g) {
  size_t total = 0;
  carve(g, nullptr, &total);
  return total;
}

hipError_t launch_linear(const KGeom& g, const uint16_t* qc, const uint16_t* kc, const uint16_t* vt,
                         const int32_t* idx, int topk, const float* o_sparse, uint16_t* oc, void* ws,
                         hipStream_t s) {
  const LinWs w = carve(g, ws, nullptr);
  const int G = (g.nc + kGroup - 1) / kGroup;
  const unsigned bh = (unsigned)(g.B * g.H);
  if (g.D == 64) {
    hipLaunchKernelGGL(lin_state<64>, dim3(G, g.H, g.B), dim3(256), 0, s, kc, vt, w, g);
    hipLaunchKernelGGL(lin_reduce<64>, dim3(bh), dim3(256), 0, s, w, g);
    hipLaunchKernelGGL(lin_apply<64>, dim3(g.nc, g.H, g.B), dim3(128), 0, s, qc, vt, idx, topk, o_sparse, oc, w, g);
  } else {
    hipLaunchKernelGGL(lin_state<128>, dim3(G, g.H, g.B), dim3(256), 0, s, kc, vt, w, g);
    hipLaunchKernelGGL(lin_reduce<128>, dim3(bh), dim3(256), 0, s, w, g);
    hipLaunchKernelGGL(lin_apply<128>, dim3(g.nc, g.H, g.B), dim3(128), 0, s, qc, vt, idx, topk, o_sparse, oc, w,
                       g);
  }
  return hipGetLastError();
}

}  // namespace vsa
