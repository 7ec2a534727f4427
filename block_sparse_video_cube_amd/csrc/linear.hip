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
//   lin_state   per (b, h, group of cubes): phi(K) (bf16, padded rows 0)
//               written token-major for lin_apply, and partial
//               S = phi(K)^T V (bf16 MFMA, fp32 accumulate; phi(K)^T read
//               with the transposed LDS read) and z = sum phi(K);
//   lin_reduce  per (b, h, 256 state elements): S_tot^T split into bf16
//               hi + lo halves, z_tot;
//   lin_apply   per (b, h, query cube): num / den and the combine.
#include <math.h>

#include "tile_pipeline.h"

namespace vsa {

namespace {

using namespace tiles;
// Cubes per partial state: the groups of all (b, h) fill the resident
// workgroup slots of lin_state (two per CU on the 256 CUs) in one round,
// which also keeps the partial-state traffic small.
struct LinGroups {
  int size;   // cubes per group
  int count;  // groups per (b, h)
};
constexpr int kStateSlots = 2 * 256;
__host__ __device__ inline LinGroups lin_groups(const KGeom& g) {
  const int bh = g.B * g.H;
  const int want = bh >= kStateSlots ? 1 : kStateSlots / bh;
  const int size = (g.nc + want - 1) / want;
  return LinGroups{size, (g.nc + size - 1) / size};
}

__device__ __forceinline__ float phi(float x) { return phi_elu1(x); }

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
  const size_t G = lin_groups(g).count;
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

// Per cube of the group: phi(K) goes to HBM (token-major, for lin_apply) and
// to one of two LDS slots (token-major, kt_swz), from which each wavefront
// reads phi(K)^T fragments with the transposed LDS read; the V^T tile goes
// to an LDS slot too (v_swz layout) for the B operands.  Each thread loads
// its share of the next cube's K and V^T rows while the current cube's
// products run, and one barrier per cube orders the slots.  Wavefront w owns
// state rows d = 32 mt .. +31 and NT column tiles.
template <int D>
__global__ void __launch_bounds__(256, 2) lin_state(const uint16_t* __restrict__ kc, const uint16_t* __restrict__ vt,
                                                    LinWs ws, KGeom g) {
  constexpr int CH = D / 8;              // 16-byte chunks per row
  constexpr int PT = 64 * CH / 256;      // chunks per thread per tile
  constexpr int RGS = 256 / CH;          // threads sharing one d chunk
  constexpr int NT = (D == 128) ? 4 : 1; // e tiles per wave
  __shared__ __attribute__((aligned(16))) uint16_t fks[2][64 * D];
  __shared__ __attribute__((aligned(16))) uint16_t vts[2][D * 64];
  __shared__ float zred[RGS][D];
  const int grp = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, hf = lane >> 5, n = lane & 31;
  const long long bh = (long long)b * g.H + h;
  const LinGroups lg = lin_groups(g);
  const int G = lg.count;
  const int mt = (D == 128) ? w : (w >> 1);
  const int nt0 = (D == 128) ? 0 : (w & 1);
  const int ch = tid % CH;
  const int c0 = grp * lg.size, c1 = min(g.nc, c0 + lg.size);
  f32x16 acc[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) acc[t] = f32x16{};
  float zacc[8] = {};

  uint4 kreg[PT], vreg[PT];
  auto load = [&](int c) {
    const uint4* ksrc = reinterpret_cast<const uint4*>(kc + (bh * g.Np + 64LL * c) * D);
    const uint4* vsrc = reinterpret_cast<const uint4*>(vt + (bh * g.Np + 64LL * c) * D);
#pragma unroll
    for (int p = 0; p < PT; ++p) {
      kreg[p] = ksrc[tid + 256 * p];
      vreg[p] = vsrc[tid + 256 * p];
    }
  };
  load(c0);
  for (int c = c0; c < c1; ++c) {
    const int slot = (c - c0) & 1;
    int ct, cy, cx;
    cube_coords(g, c, ct, cy, cx);
    uint4* fdst = reinterpret_cast<uint4*>(ws.fk + (bh * g.Np + 64LL * c) * D);
#pragma unroll
    for (int p = 0; p < PT; ++p) {
      const int f = tid + 256 * p, row = f / CH;
      const bool valid = local_valid(g, ct, cy, cx, row);
      const uint32_t wv[4] = {kreg[p].x, kreg[p].y, kreg[p].z, kreg[p].w};
      uint32_t outw[4];
#pragma unroll
      for (int e2 = 0; e2 < 4; ++e2) {
        const float x0 = __uint_as_float(wv[e2] << 16), x1 = __uint_as_float(wv[e2] & 0xFFFF0000u);
        const uint16_t p0 = valid ? f32_to_bf16(phi(x0)) : 0, p1 = valid ? f32_to_bf16(phi(x1)) : 0;
        zacc[2 * e2] += bf16_to_f32(p0);
        zacc[2 * e2 + 1] += bf16_to_f32(p1);
        outw[e2] = (uint32_t)p0 | ((uint32_t)p1 << 16);
      }
      const uint4 o = make_uint4(outw[0], outw[1], outw[2], outw[3]);
      fdst[f] = o;
      *reinterpret_cast<uint4*>(&fks[slot][row * D + ((ch ^ kt_swz<D>(row)) << 3)]) = o;
      // V^T row e = f / 8 (64 tokens, 8 chunks of 8).
      const int vrow = f >> 3, vch = f & 7;
      *reinterpret_cast<uint4*>(&vts[slot][vrow * 64 + ((vch ^ v_swz(vrow)) << 3)]) = vreg[p];
    }
    if (c + 1 < c1) load(c + 1);
    pipeline_barrier();  // this cube's slots are complete; the slots written next were last read two cubes ago
#pragma unroll
    for (int wk = 0; wk < 2; ++wk) {
      bf16x8 va[D / 32][2];
      read_v<D>(vts[slot], wk, hf, n, va);
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const bf16x8 a = read_tr_one<D>(fks[slot], 32 * wk + 16 * kk, mt, lane);
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          // D = 64: one column tile per wave, picked by the uniform nt0.
          const bf16x8 bop = (D == 128) ? va[t][kk] : (nt0 ? va[D / 32 - 1][kk] : va[0][kk]);
          acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bop, acc[t], 0, 0, 0);
        }
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

// One thread per state element (d, e) of one (b, h): sums the group partials
// (coalesced across threads) and writes S_tot^T as bf16 hi + lo.  Workgroup
// (chunk, bh) covers 256 consecutive elements; the last chunk also sums z.
template <int D>
__global__ void __launch_bounds__(256) lin_reduce(LinWs ws, KGeom g) {
  const long long bh = blockIdx.y;
  const int G = lin_groups(g).count;
  const int f = blockIdx.x * 256 + threadIdx.x;  // < D * D
  const float* sp = ws.s_part + bh * G * (long long)D * D;
  float s = 0.f;
#pragma unroll 8
  for (int gi = 0; gi < G; ++gi) s += sp[(long long)gi * D * D + f];
  const int d = f / D, e = f % D;
  const uint16_t hi = f32_to_bf16(s);
  const uint16_t lo = f32_to_bf16(s - bf16_to_f32(hi));
  ws.st_hi[bh * D * D + e * D + d] = hi;
  ws.st_lo[bh * D * D + e * D + d] = lo;
  if (blockIdx.x == gridDim.x - 1 && threadIdx.x < D) {
    float z = 0.f;
    for (int gi = 0; gi < G; ++gi) z += ws.z_part[(bh * G + gi) * D + threadIdx.x];
    ws.z_tot[bh * D + threadIdx.x] = z;
  }
}

// Three phi(K) and two V^T tile buffers (80 KB at D = 128).
template <int D>
struct LinSmem {
  uint16_t f[3][64 * D];
  uint16_t v[2][D * 64];
};

// One workgroup per (b, h, query cube), the same wavefront split and tile
// pipeline as the fine stage: wavefront (wq, wk) owns queries 32 wq .. +31 and
// keys 32 wk .. +31 of every selected block.  Per block it forms
// A^T = phi(K) phi(Q)^T on the matrix cores, rounds A to bf16 (its row sums,
// taken on the same rounded values, go to the denominator) and accumulates
// V^T A^T.  The total part phi(Q) S_tot is split between the two key halves
// (bf16 hi half on wk = 0, lo half on wk = 1) so that the merge through LDS
// adds num - corr directly.
//
// BWD: instead of the combine, the per-row inputs of the linear branch's
// backward: w = dO / den (bf16), c = (dO . O_lin) / den (fp32) and phi(Q)
// (bf16), zero on padded query rows and when no cube is left unselected.
template <int D, bool BWD>
__global__ void __launch_bounds__(kThreads, 2) lin_apply(const uint16_t* __restrict__ qc,
                                                         const uint16_t* __restrict__ vt,
                                                         const int32_t* __restrict__ idx, int topk,
                                                         const float* __restrict__ o_sparse,
                                                         uint16_t* __restrict__ oc, LinWs ws, KGeom g,
                                                         Placement pl, LinBwdRows br) {
  constexpr int DC = D / 16, DT = D / 32;
  __shared__ __attribute__((aligned(16))) LinSmem<D> sm;
  int i, h, b;
  if (!map_workgroup(g, pl, i, h, b)) return;  // whole workgroup leaves before any barrier
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wq = w & 1, wk = w >> 1;
  const int hf = lane >> 5, n = lane & 31;
  const long long bh = (long long)b * g.H + h;
  const int q = 32 * wq + n;
  const long long row = bh * g.Np + 64LL * i + q;
  const bool empty_u = topk >= g.nc;  // every cube selected: O_lin = 0
  const int32_t* irow = idx + (bh * g.nc + i) * topk;
  const uint16_t* fkb = ws.fk + bh * g.Np * D;
  const uint16_t* vb = vt + bh * g.Np * D;
  const TileOffsets<D> toff(w, lane);
  // phiK(0), V(0) and phiK(1); past the end of the list (or with no
  // unselected cube) a zero-size range, so every step issues the same loads.
  constexpr unsigned kTile = 64 * D * 2;
  issue_k_tile<D>(make_rsrc(fkb + 64LL * irow[0] * D, empty_u ? 0 : kTile), sm.f[0], w, toff.k);
  issue_v_tile<D>(make_rsrc(vb + 64LL * irow[0] * D, empty_u ? 0 : kTile), sm.v[0], w, toff.v);
  issue_k_tile<D>(make_rsrc(fkb + 64LL * irow[topk > 1 ? 1 : 0] * D, (empty_u || topk < 2) ? 0 : kTile), sm.f[1], w,
                  toff.k);

  // phi(Q) fragments (bf16) and this lane's part of phi(Q) . z_tot.
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
      __builtin_amdgcn_sched_barrier(0);  // one chunk of loads at a time (register budget)
    }
  }

  // c starts as this key half's share of phi(Q) S_tot (the hi or the lo
  // half), computed while the first tiles arrive; the loop below subtracts
  // the selected part by feeding the products exactly negated weights.
  f32x16 c[DT];
  {
    const uint16_t* st = (wk == 0 ? ws.st_hi : ws.st_lo) + bh * D * D;
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

  // Selected part, block by block.
  float dcorr = 0.f;
  const int prow = pi_row(n);
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
  // phiK runs two blocks ahead (three buffers), V one (two buffers); steps
  // come in groups of six so that every buffer index is compile-time.
  for (int jb = 0; jb < (empty_u ? 0 : topk); jb += 6) {
#pragma unroll
    for (int u = 0; u < 6; ++u) {
      const int nb = jb + u;
      if (nb < topk) {
        // Outstanding, oldest first: phiK(nb), V(nb), phiK(nb+1).
        wait_vmcnt<TileOffsets<D>::NI>();
        pipeline_barrier();
        issue_v_tile<D>(make_rsrc(vb + 64LL * irow[nb + 1 < topk ? nb + 1 : nb] * D, nb + 1 < topk ? kTile : 0),
                        sm.v[(u + 1) % 2], w, toff.v);
        issue_k_tile<D>(make_rsrc(fkb + 64LL * irow[nb + 2 < topk ? nb + 2 : nb] * D, nb + 2 < topk ? kTile : 0),
                        sm.f[(u + 2) % 3], w, toff.k);
        bf16x8 ka[DC];
        bf16x8 va[DT][2];
        read_k<D>(sm.f[u % 3], wk, hf, prow, ka);
        read_v<D>(sm.v[u % 2], wk, hf, n, va);
        f32x16 sa = f32x16{};
#pragma unroll
        for (int dc = 0; dc < DC; ++dc) sa = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[dc], fq[dc], sa, 0, 0, 0);
        uint32_t pw[8];
#pragma unroll
        for (int r = 0; r < 8; ++r) {
          const bf16x2 pk = __builtin_convertvector((f32x2){sa[2 * r], sa[2 * r + 1]}, bf16x2);
          dcorr = __builtin_amdgcn_fdot2_f32_bf16(pk, ones, dcorr, false);
          pw[r] = __builtin_bit_cast(uint32_t, pk) ^ 0x80008000u;  // -P' (exact in bf16)
        }
        bf16x8 pb[2];
        pb[0] = __builtin_bit_cast(bf16x8, make_uint4(pw[0], pw[1], pw[2], pw[3]));
        pb[1] = __builtin_bit_cast(bf16x8, make_uint4(pw[4], pw[5], pw[6], pw[7]));
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
          for (int kk = 0; kk < 2; ++kk)
            c[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[dt][kk], pb[kk], c[dt], 0, 0, 0);
      }
    }
  }

  // Merge the two key halves through LDS.
  dcorr += __shfl_xor(dcorr, 32);
  wait_vmcnt<0>();  // the last steps' zero-size loads land in f[] and v[] too
  __syncthreads();  // every tile read has completed; reuse the tile buffers
  float* xo = reinterpret_cast<float*>(&sm.f[0][0]) + wq * (DT * 16 * 64);
  float* xd = reinterpret_cast<float*>(&sm.v[0][0]) + wq * 64;
  if (wk == 1) {
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) xo[(dt * 16 + r) * 64 + lane] = c[dt][r];
    xd[lane] = dcorr;
  }
  __syncthreads();
  if (wk == 1) return;
  const float den = (den_part + __shfl_xor(den_part, 32)) - (dcorr + xd[lane]);
  const float inv = empty_u ? 0.f : 1.f / den;
  if (BWD) {
    int ct, cy, cx;
    cube_coords(g, i, ct, cy, cx);
    const float inv_b = local_valid(g, ct, cy, cx, q) ? inv : 0.f;
    const uint16_t* dsrc = br.doc + row * D;
    uint16_t* wdst = br.w + row * D;
    float cp = 0.f;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        const int e = 32 * dt + 8 * gq + 4 * hf;
        const uint2 draw = *reinterpret_cast<const uint2*>(dsrc + e);
        const float dov[4] = {__uint_as_float(draw.x << 16), __uint_as_float(draw.x & 0xFFFF0000u),
                              __uint_as_float(draw.y << 16), __uint_as_float(draw.y & 0xFFFF0000u)};
        // c is taken from the same bf16-rounded w that the backward's
        // products use, so that S_U w and c z_U, which nearly cancel, carry
        // the same rounding.
        const uint2 wbits = make_uint2(pack_bf16x2(dov[0] * inv_b, dov[1] * inv_b),
                                       pack_bf16x2(dov[2] * inv_b, dov[3] * inv_b));
        const float wr[4] = {__uint_as_float(wbits.x << 16), __uint_as_float(wbits.x & 0xFFFF0000u),
                             __uint_as_float(wbits.y << 16), __uint_as_float(wbits.y & 0xFFFF0000u)};
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int r = 4 * gq + u;
          const float olin = (c[dt][r] + xo[(dt * 16 + r) * 64 + lane]) * inv;
          cp = fmaf(wr[u], olin, cp);
        }
        *reinterpret_cast<uint2*>(wdst + e) = wbits;
      }
    cp += __shfl_xor(cp, 32);
    if (hf == 0) br.c[row] = cp;
#pragma unroll
    for (int dc = 0; dc < DC; ++dc)
      *reinterpret_cast<bf16x8*>(br.fq + row * D + 16 * dc + 8 * hf) = inv_b != 0.f ? fq[dc] : bf16x8{};
    return;
  }
  const float* osrc = o_sparse + row * D;
  uint16_t* odst = oc + row * D;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int gq = 0; gq < 4; ++gq) {
      const int e = 32 * dt + 8 * gq + 4 * hf;
      const float4 os = *reinterpret_cast<const float4*>(osrc + e);
      float v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int r = 4 * gq + u;
        v[u] = (c[dt][r] + xo[(dt * 16 + r) * 64 + lane]) * inv;
      }
      *reinterpret_cast<uint2*>(odst + e) =
          make_uint2(pack_bf16x2(os.x + v[0], os.y + v[1]), pack_bf16x2(os.z + v[2], os.w + v[3]));
    }
}

}  // namespace

size_t linear_workspace_bytes(const KGeom& g) {
  size_t total = 0;
  carve(g, nullptr, &total);
  return total;
}

LinTensors lin_tensors(const KGeom& g, void* ws) {
  const LinWs w = carve(g, ws, nullptr);
  return LinTensors{w.fk, w.st_hi, w.st_lo, w.z_tot};
}

hipError_t launch_lin_prep(const KGeom& g, const uint16_t* kc, const uint16_t* vt, void* ws, hipStream_t s) {
  const LinWs w = carve(g, ws, nullptr);
  const int G = lin_groups(g).count;
  const unsigned bh = (unsigned)(g.B * g.H);
  if (g.D == 64) {
    hipLaunchKernelGGL(lin_state<64>, dim3(G, g.H, g.B), dim3(256), 0, s, kc, vt, w, g);
    hipLaunchKernelGGL(lin_reduce<64>, dim3(64 * 64 / 256, bh), dim3(256), 0, s, w, g);
  } else {
    hipLaunchKernelGGL(lin_state<128>, dim3(G, g.H, g.B), dim3(256), 0, s, kc, vt, w, g);
    hipLaunchKernelGGL(lin_reduce<128>, dim3(128 * 128 / 256, bh), dim3(256), 0, s, w, g);
  }
  return hipGetLastError();
}

hipError_t launch_linear(const KGeom& g, const uint16_t* qc, const uint16_t* kc, const uint16_t* vt,
                         const int32_t* idx, int topk, const float* o_sparse, uint16_t* oc, void* ws,
                         hipStream_t s) {
  hipError_t e = launch_lin_prep(g, kc, vt, ws, s);
  if (e != hipSuccess) return e;
  const LinWs w = carve(g, ws, nullptr);
  const LinBwdRows none{};
  if (g.D == 64)
    hipLaunchKernelGGL((lin_apply<64, false>), dim3(grid_size(g)), dim3(kThreads), 0, s, qc, vt, idx, topk,
                       o_sparse, oc, w, g, make_placement(g), none);
  else
    hipLaunchKernelGGL((lin_apply<128, false>), dim3(grid_size(g)), dim3(kThreads), 0, s, qc, vt, idx, topk,
                       o_sparse, oc, w, g, make_placement(g), none);
  return hipGetLastError();
}

hipError_t launch_lin_bwd_rows(const KGeom& g, const uint16_t* qc, const uint16_t* vt, const int32_t* idx, int topk,
                               const LinBwdRows& br, void* ws, hipStream_t s) {
  const LinWs w = carve(g, ws, nullptr);
  if (g.D == 64)
    hipLaunchKernelGGL((lin_apply<64, true>), dim3(grid_size(g)), dim3(kThreads), 0, s, qc, vt, idx, topk, nullptr,
                       nullptr, w, g, make_placement(g), br);
  else
    hipLaunchKernelGGL((lin_apply<128, true>), dim3(grid_size(g)), dim3(kThreads), 0, s, qc, vt, idx, topk,
                       nullptr, nullptr, w, g, make_placement(g), br);
  return hipGetLastError();
}

LinState lin_state_parts(const KGeom& g, void* ws) {
  const LinWs w = carve(g, ws, nullptr);
  const LinGroups lg = lin_groups(g);
  return LinState{w.fk, w.s_part, w.z_part, w.z_tot, lg.size, lg.count};
}

}  // namespace vsa
