// Linear branch through per-cube states (the sparse branch's partner: a
// low-rank linear attention over the blocks the top-k left out, SparkDiffusion
// article, paragraph 3, RoLA; TurboDiffusion article, section
// "稀疏、蒸馏与全链路量化", SLA).
//
// For query cube i with unselected key cubes U(i) the branch is
//   O_lin = phi(Q_i) S_U(i) / (phi(Q_i) . z_U(i)),  phi = elu + 1,
//   S_U(i) = sum_{j in U(i)} S_j,  S_j = phi(K_j)^T V_j,  z_U(i) = sum_{j in U(i)} z_j,
// z_j the column sums of phi(K_j).  A cube's state S_j (D x D) holds exactly
// as many values as its K and V tiles together (64 x D each), so instead of
// streaming tiles per selected block this path sums states:
//   1. lin_cube_states: S_j and z_j of every key cube (bf16);
//   2. lin_sel_bits + lin_unsel_sum: S_U(i), z_U(i) for every query cube i
//      as one dense product U . [S_j, z_j] per head, U the 0/1 matrix of
//      unselected pairs.  The dense form spends 2 Nc flops per state value,
//      a fraction Nc / (64 k) of the tile path's 4 * 64 * 64 * D flops per
//      selected block (k the blocks per row), and reads each state tile once
//      per 128 query cubes instead of once per selection; U is exact in
//      bf16, the sum runs in fp32;
//   3. the fine stage's epilogue applies phi(Q_i) to S_U(i) and z_U(i)
//      (attn_fwd.hip, LIN), so O_sparse never leaves registers.
// U is taken directly (no total minus selected), so nothing cancels.
#include "common.h"
#include "tile_pipeline.h"

namespace vsa {

namespace {

using namespace tiles;

constexpr int kSumThreads = 256;
constexpr int kSumRange = 128;  // query cubes per lin_unsel_sum workgroup (4 wavefronts x 32)

// States of every key cube of one group (lin_groups sizing: all groups of all
// heads in one round of two workgroups per compute unit).  Per cube, phi(K)
// goes to an LDS slot (token-major, kt_swz; padded key rows zero) and V^T to
// another (v_swz); wavefront w owns state rows d = 32 mt .. +31 (phi
// features) and NT column tiles e (value dims), plus, from a B operand of
// ones, the column sums z[d].  Output st [B, H, D + 1, Nc, D] bf16:
// st[bh][e][j][d] = S_j[d][e] for e < D, st[bh][D][j][d] = z_j[d], so that
// 64 cubes x D values of one e are one contiguous 16 KB tile for
// lin_unsel_sum.  The next cube's K and V^T rows are loaded into registers
// while the current cube's products run; one barrier per cube.
template <int D>
__global__ void __launch_bounds__(256, 2) lin_cube_states(const uint16_t* __restrict__ kc,
                                                          const uint16_t* __restrict__ vt,
                                                          uint16_t* __restrict__ st, KGeom g, int gsize) {
  constexpr int CH = D / 8;              // 16-byte chunks per row
  constexpr int PT = 64 * CH / 256;      // chunks per thread per tile
  constexpr int NT = (D == 128) ? 4 : 1; // e tiles per wave
  __shared__ __attribute__((aligned(16))) uint16_t fks[2][64 * D];
  __shared__ __attribute__((aligned(16))) uint16_t vts[2][D * 64];
  const int grp = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, hf = lane >> 5, n = lane & 31;
  const long long bh = (long long)b * g.H + h;
  const int mt = (D == 128) ? w : (w >> 1);
  const int nt0 = (D == 128) ? 0 : (w & 1);
  const bool zw = nt0 == 0;  // wavefronts that also form z (wave-uniform)
  const int ch = tid % CH;
  const int c0 = grp * gsize, c1 = min(g.nc, c0 + gsize);
  if (c0 >= c1) return;
  const bf16x2 one2 = {(__bf16)1.0f, (__bf16)1.0f};
  const bf16x8 ones = __builtin_shufflevector(one2, one2, 0, 1, 0, 1, 0, 1, 0, 1);
  const long long xs = (long long)g.nc * D;  // elements between consecutive e of one head

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
#pragma unroll
    for (int p = 0; p < PT; ++p) {
      const int f = tid + 256 * p, row = f / CH;
      const bool valid = local_valid(g, ct, cy, cx, row);
      const uint4 o = valid ? make_uint4(phi2_bf16(kreg[p].x), phi2_bf16(kreg[p].y), phi2_bf16(kreg[p].z),
                                         phi2_bf16(kreg[p].w))
                            : make_uint4(0, 0, 0, 0);
      *reinterpret_cast<uint4*>(&fks[slot][row * D + ((ch ^ kt_swz<D>(row)) << 3)]) = o;
      const int vrow = f >> 3, vch = f & 7;  // V^T row (64 tokens, 8 chunks of 8)
      *reinterpret_cast<uint4*>(&vts[slot][vrow * 64 + ((vch ^ v_swz(vrow)) << 3)]) = vreg[p];
    }
    if (c + 1 < c1) load(c + 1);
    pipeline_barrier();  // this cube's slots are complete; the slots written next were last read two cubes ago
    f32x16 acc[NT], az = f32x16{};
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[t] = f32x16{};
#pragma unroll
    for (int wk = 0; wk < 2; ++wk) {
      bf16x8 va[D / 32][2];
      read_v<D>(vts[slot], wk, hf, n, va);
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const bf16x8 a = read_tr_one<D>(fks[slot], 32 * wk + 16 * kk, mt, lane);
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          const bf16x8 bop = (D == 128) ? va[t][kk] : (nt0 ? va[D / 32 - 1][kk] : va[0][kk]);
          acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bop, acc[t], 0, 0, 0);
        }
        if (zw) az = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, ones, az, 0, 0, 0);
      }
    }
    // acc[t][r]: S[d][e], d = 32 mt + 8 (r/4) + 4 hf + r%4, e = 32 (nt0 + t) + n;
    // four consecutive d per lane and group go out as one 8-byte store.
    uint16_t* sc = st + (bh * (D + 1)) * xs + (long long)c * D;
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        const int d = 32 * mt + 8 * gq + 4 * hf, e = 32 * (nt0 + t) + n;
        *reinterpret_cast<uint2*>(sc + e * xs + d) =
            make_uint2(pack_bf16x2(acc[t][4 * gq], acc[t][4 * gq + 1]), pack_bf16x2(acc[t][4 * gq + 2], acc[t][4 * gq + 3]));
      }
    if (zw && n == 0) {
      // Every column of az holds z[d] for this wavefront's rows.
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        const int d = 32 * mt + 8 * gq + 4 * hf;
        *reinterpret_cast<uint2*>(sc + D * xs + d) =
            make_uint2(pack_bf16x2(az[4 * gq], az[4 * gq + 1]), pack_bf16x2(az[4 * gq + 2], az[4 * gq + 3]));
      }
    }
  }
}

// Selection bits: bits[row][w] has bit t set when cube 32 w + t is in the
// row's list (one thread per row; entries need not be sorted; an entry
// outside 0..Nc-1 selects nothing).
__global__ void __launch_bounds__(256) lin_sel_bits(const int32_t* __restrict__ idx, int topk,
                                                    uint32_t* __restrict__ bits, int nc, int nwords,
                                                    long long nrows) {
  const long long row = (long long)blockIdx.x * 256 + threadIdx.x;
  if (row >= nrows) return;
  uint32_t* out = bits + row * nwords;
  for (int w = 0; w < nwords; ++w) out[w] = 0u;
  const int32_t* irow = idx + row * topk;
  for (int m = 0; m < topk; ++m) {
    const int j = irow[m];
    if ((unsigned)j < (unsigned)nc) out[j >> 5] |= 1u << (j & 31);
  }
}

// Work item of lin_unsel_sum: (b, h), state column xc (0..D: value dim e, or
// D for z) and a range of 128 query cubes.  Items run in the order (bh, xc,
// range) with consecutive items on one XCD (workgroup id = 8 slot + XCD), so
// the ranges that read the same state column share its tiles in that L2.
struct SumPlace {
  int ranges;   // query-cube ranges per (bh, xc)
  int items;    // B * H * (D + 1) * ranges
  int per_xcd;  // items per XCD
};

inline SumPlace make_sum_place(const KGeom& g) {
  SumPlace p;
  p.ranges = (g.nc + kSumRange - 1) / kSumRange;
  p.items = g.B * g.H * (g.D + 1) * p.ranges;
  p.per_xcd = (p.items + 7) / 8;
  return p;
}

// S_U and z_U of every query cube: out[bh][i][xc][d] = sum_j U[i][j] st[bh][xc][j][d]
// over j < Nc, with U[i][j] = 1 when j is not in row i's list.  On the
// matrix cores as out^T = st^T U^T: the A operand (32 d x 16 j) comes from a
// 64-cube state tile in LDS read transposed (ds_read_b64_tr_b16), the B
// operand (16 j x 32 i) from the selection bits in registers.  Wavefront w
// owns query cubes 32 w .. +31 of the range and all D / 32 row tiles of d.
// Tiles of 64 cubes are double-buffered; rows past Nc read as zero (the
// buffer range ends at Nc).  Output su [B, H, Nc, D * D + D] bf16: for query
// cube i, su[e * D + d] = S_U[d][e] and su[D * D + d] = z_U[d].
template <int D>
__global__ void __launch_bounds__(kSumThreads, 2) lin_unsel_sum(const uint16_t* __restrict__ st,
                                                                const uint32_t* __restrict__ bits,
                                                                uint16_t* __restrict__ su, KGeom g, int nwords,
                                                                SumPlace pl) {
  constexpr int DT = D / 32;
  __shared__ __attribute__((aligned(16))) uint16_t tl[2][64 * D];
  const int item = (blockIdx.x & 7) * pl.per_xcd + (blockIdx.x >> 3);
  if (item >= pl.items) return;  // whole workgroup leaves before any barrier
  const int rg = item % pl.ranges, rest = item / pl.ranges;
  const int xc = rest % (D + 1);
  const long long bh = rest / (D + 1);
  const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hf = lane >> 5, n = lane & 31;
  const int i = rg * kSumRange + 32 * w + n;  // this lane's query cube (B column)
  const bool ivalid = i < g.nc;
  const uint32_t* brow = bits + (bh * g.nc + (ivalid ? i : 0)) * nwords;
  const uint16_t* sbase = st + (bh * (D + 1) + xc) * (long long)g.nc * D;
  const TileOffsets<D, true> toff(w, lane);
  const int ntl = (g.nc + 63) / 64;
  const auto rsrc = [&](int t) {
    const int rows = min(64, g.nc - 64 * t);
    return make_rsrc(sbase + 64LL * t * D, (unsigned)(rows * D * 2));
  };
  // The two selection words of tile t (cubes 64 t .. +63).
  const auto words = [&](int t) {
    const uint32_t w0 = brow[2 * t];
    const uint32_t w1 = (2 * t + 1 < nwords) ? brow[2 * t + 1] : 0xFFFFFFFFu;
    return make_uint2(w0, w1);
  };
  issue_k_tile<D>(rsrc(0), tl[0], w, toff.k);
  uint2 wcur = words(0);
  f32x16 acc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) acc[dt] = f32x16{};
  for (int t = 0; t < ntl; ++t) {
    wait_vmcnt<0>();
    pipeline_barrier();  // tile t is in; the other slot was last read in step t - 1
    // The next tile's selection words are loaded before its tile, so that
    // waiting for them leaves the tile loads in flight.
    uint2 wnext = wcur;
    if (t + 1 < ntl) {
      wnext = words(t + 1);
      issue_k_tile<D>(rsrc(t + 1), tl[(t + 1) & 1], w, toff.k);
    }
    const uint16_t* slot = tl[t & 1];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      // Cubes 64 t + 16 ks + 8 hf + e, e = 0..7: U = 1 where the bit is clear.
      const uint32_t sel = ((ks < 2) ? wcur.x : wcur.y) >> (16 * (ks & 1) + 8 * hf);
      const uint32_t u = ivalid ? (~sel & 0xFFu) : 0u;
      uint32_t bw[4];
#pragma unroll
      for (int e2 = 0; e2 < 4; ++e2)
        bw[e2] = (((u >> (2 * e2)) & 1u) ? 0x3F80u : 0u) | (((u >> (2 * e2 + 1)) & 1u) ? 0x3F800000u : 0u);
      const bf16x8 bop = __builtin_bit_cast(bf16x8, make_uint4(bw[0], bw[1], bw[2], bw[3]));
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const bf16x8 a = read_tr_one<D>(slot, 16 * ks, dt, lane);
        acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bop, acc[dt], 0, 0, 0);
      }
    }
    wcur = wnext;
  }
  if (!ivalid) return;
  uint16_t* orow = su + (bh * g.nc + i) * (long long)(D * D + D) + xc * D;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int gq = 0; gq < 4; ++gq) {
      const int d = 32 * dt + 8 * gq + 4 * hf;
      *reinterpret_cast<uint2*>(orow + d) = make_uint2(pack_bf16x2(acc[dt][4 * gq], acc[dt][4 * gq + 1]),
                                                       pack_bf16x2(acc[dt][4 * gq + 2], acc[dt][4 * gq + 3]));
    }
}

// Groups of cubes for lin_cube_states: enough groups that all (b, h) fill two
// workgroups per compute unit in one round.
inline int state_group_size(const KGeom& g) {
  const int bh = g.B * g.H;
  const int want = bh >= 512 ? 1 : 512 / bh;
  return (g.nc + want - 1) / want;
}

}  // namespace

size_t linear_states_bytes(const KGeom& g) {
  return (size_t)g.B * g.H * (g.D + 1) * (size_t)g.nc * g.D * 2;
}

size_t linear_unsel_bytes(const KGeom& g) {
  return (size_t)g.B * g.H * (size_t)g.nc * ((size_t)g.D * g.D + g.D) * 2;
}

size_t linear_unsel_workspace_bytes(const KGeom& g) {
  const size_t nwords = ((size_t)g.nc + 31) / 32;
  return ((size_t)g.B * g.H * g.nc * nwords * 4 + 255) / 256 * 256;
}

hipError_t launch_lin_cube_states(const KGeom& g, const uint16_t* kc, const uint16_t* vt, uint16_t* st,
                                  hipStream_t s) {
  const int gs = state_group_size(g);
  const dim3 grid((unsigned)((g.nc + gs - 1) / gs), g.H, g.B);
  if (g.D == 64) hipLaunchKernelGGL(lin_cube_states<64>, grid, dim3(256), 0, s, kc, vt, st, g, gs);
  else hipLaunchKernelGGL(lin_cube_states<128>, grid, dim3(256), 0, s, kc, vt, st, g, gs);
  return hipGetLastError();
}

hipError_t launch_lin_unselected(const KGeom& g, const uint16_t* st, const int32_t* idx, int topk, uint16_t* su,
                                 void* ws, hipStream_t s) {
  uint32_t* bits = static_cast<uint32_t*>(ws);
  const int nwords = (g.nc + 31) / 32;
  const long long nrows = (long long)g.B * g.H * g.nc;
  lin_sel_bits<<<dim3((unsigned)((nrows + 255) / 256)), dim3(256), 0, s>>>(idx, topk, bits, g.nc, nwords, nrows);
  const SumPlace pl = make_sum_place(g);
  const dim3 grid((unsigned)(8 * pl.per_xcd));
  if (g.D == 64) hipLaunchKernelGGL(lin_unsel_sum<64>, grid, dim3(kSumThreads), 0, s, st, bits, su, g, nwords, pl);
  else hipLaunchKernelGGL(lin_unsel_sum<128>, grid, dim3(kSumThreads), 0, s, st, bits, su, g, nwords, pl);
  return hipGetLastError();
}

}  // namespace vsa
