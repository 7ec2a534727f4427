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
#include <algorithm>
#include <type_traits>

#include "common.h"
#include "tile_pipeline.h"

namespace vsa {

namespace {

using namespace tiles;

// Two fp32 values to two bf16 (one v_cvt_pk_bf16_f32, round to nearest even).
__device__ __forceinline__ uint32_t cvt2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){lo, hi}, bf16x2));
}

constexpr int kSumThreads = 256;
// Query cubes per lin_unsel_sum workgroup: 4 wavefronts x NT column tiles of 32.
template <int NT>
constexpr int sum_range() { return 4 * 32 * NT; }

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

// Selection bits of every row (b, h, i), tile-major: bits[bh][t][i] is the
// pair of words for cubes 64 t .. 64 t + 63 of row i, bit b of word h set
// when cube 64 t + 32 h + b is in the row's list (one thread per row; entries
// need not be sorted; an entry outside 0..Nc-1 selects nothing; bits past Nc
// are set, so no cube there is summed).  One tile's words of 256 consecutive
// rows are 2 KB in a row, loaded beside the state tile.
__global__ void __launch_bounds__(256) lin_sel_bits(const int32_t* __restrict__ idx, int topk,
                                                    uint2* __restrict__ bits, int nc, int ntl, long long nrows) {
  const long long row = (long long)blockIdx.x * 256 + threadIdx.x;
  if (row >= nrows) return;
  const long long bh = row / nc;
  const int i = (int)(row - bh * nc);
  uint2* out = bits + bh * ntl * (long long)nc + i;
  const auto pad = [&](int lo) {
    return lo + 32 <= nc ? 0u : (lo >= nc ? 0xFFFFFFFFu : (0xFFFFFFFFu << (nc - lo)));
  };
  for (int t = 0; t < ntl; ++t) out[(long long)t * nc] = make_uint2(pad(64 * t), pad(64 * t + 32));
  const int32_t* irow = idx + row * topk;
  for (int m = 0; m < topk; ++m) {
    const int j = irow[m];
    if ((unsigned)j >= (unsigned)nc) continue;
    uint2& wp = out[(long long)(j >> 6) * nc];
    if (j & 32) wp.y |= 1u << (j & 31);
    else wp.x |= 1u << (j & 31);
  }
}

// Work item of lin_unsel_sum: (b, h), a run of `xcr` consecutive state
// columns xc (0..D: value dim e, or D for z) and a range of query cubes.  The
// run keeps one workgroup's tile pipeline going across its columns (one
// prologue per run); its length is chosen so that the items number about
// `want` (a few workgroups per compute unit).  Items run in the order (bh, run,
// range) with consecutive items on one XCD (workgroup id = 8 slot + XCD), so
// the ranges that read the same state columns share its tiles in that L2.
struct SumPlace {
  int ranges;   // query-cube ranges per (bh, run)
  int xcr;      // state columns per run
  int runs;     // runs per bh
  int items;    // B * H * runs * ranges
  int per_xcd;  // items per XCD
};

template <int NT>
inline SumPlace make_sum_place(const KGeom& g, long long want) {
  SumPlace p;
  p.ranges = (g.nc + sum_range<NT>() - 1) / sum_range<NT>();
  const long long per_col = (long long)g.B * g.H * p.ranges;
  p.xcr = (int)std::max(1LL, std::min<long long>(g.D + 1, (per_col * (g.D + 1) + want - 1) / want));
  p.runs = (g.D + 1 + p.xcr - 1) / p.xcr;
  p.items = (int)(per_col * p.runs);
  p.per_xcd = (p.items + 7) / 8;
  return p;
}

// S_U and z_U of every query cube: out[bh][i][xc][d] = sum_j U[i][j] st[bh][xc][j][d]
// over j < Nc, with U[i][j] = 1 when j is not in row i's list.  On the
// matrix cores as out^T = st^T U^T: the A operand (32 d x 16 j) comes from a
// 64-cube state tile in LDS read transposed (ds_read_b64_tr_b16), the B
// operand (16 j x 32 i) from the selection bits in registers.  Wavefront w
// owns query cubes 32 NT w .. of the range (NT column tiles of 32; a tile
// wholly past Nc is skipped) and all D / 32 row tiles of d, so each A
// operand read from LDS feeds NT products.  The workgroup streams the
// state tiles of its run of columns in one sequence (tile tau: column
// xc0 + tau / ntl, cubes 64 (tau % ntl) ..) with the range's selection
// words of those cubes, two ahead in a ring of three, and writes each
// column's sums after its last tile; rows past Nc read as zero (the buffer
// range ends at Nc).  Output su [B, H, Nc, D * D + D] bf16: for query cube
// i, su[e * D + d] = S_U[d][e] and su[D * D + d] = z_U[d].
template <int D, int NT>
__global__ void __launch_bounds__(kSumThreads, 2) lin_unsel_sum(const uint16_t* __restrict__ st,
                                                                const uint2* __restrict__ bits,
                                                                uint16_t* __restrict__ su, KGeom g, SumPlace pl) {
  constexpr int DT = D / 32, NI = TileOffsets<D, true>::NI;
  constexpr int kSumRange = sum_range<NT>(), NWI = kSumRange / 128;  // word loads per wavefront per tile
  // One LDS object per ring slot: the compiler makes a transposed LDS read
  // wait for every direct-to-LDS load in flight into the object it reads.
  // Each slot: the state tile, then the range's selection words of its cubes.
  constexpr int TW = 64 * D;  // elements of the state tile
  __shared__ __attribute__((aligned(16))) uint16_t tl0[TW + kSumRange * 4];
  __shared__ __attribute__((aligned(16))) uint16_t tl1[TW + kSumRange * 4];
  __shared__ __attribute__((aligned(16))) uint16_t tl2[TW + kSumRange * 4];
  const int item = (blockIdx.x & 7) * pl.per_xcd + (blockIdx.x >> 3);
  if (item >= pl.items) return;  // whole workgroup leaves before any barrier
  const int rg = item % pl.ranges, rest = item / pl.ranges;
  const int xc0 = (rest % pl.runs) * pl.xcr;
  const long long bh = rest / pl.runs;
  const int ncol = min(pl.xcr, D + 1 - xc0);
  const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hf = lane >> 5, n = lane & 31;
  const int ibase = rg * kSumRange + 32 * NT * w;  // this wavefront's first query cube
  // Column tiles of this wavefront that hold a real cube (a scalar count, so
  // the skip below is a uniform branch), and whether this lane's cube is real.
  const int ntv = __builtin_amdgcn_readfirstlane(min(NT, max(0, (g.nc - ibase + 31) / 32)));
  bool iv[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) iv[nt] = ibase + 32 * nt + n < g.nc;
  const TileOffsets<D, true> toff(w, lane);
  const int ntl = (g.nc + 63) / 64;
  const int ntau = ncol * ntl;
  const int nrange = min(kSumRange, g.nc - rg * kSumRange);  // rows of this range
  // Tile tau: state column xc0 + tau / ntl, cubes 64 (tau % ntl) ..; rows past
  // Nc read as zero.  Its selection words: rows of this range, tile tau % ntl.
  const auto issue = [&](int tau, uint16_t* slot) {
    const int xc = xc0 + tau / ntl, t = tau % ntl;
    const int rows = min(64, g.nc - 64 * t);
    issue_k_tile<D>(make_rsrc(st + ((bh * (D + 1) + xc) * (long long)g.nc + 64LL * t) * D, (unsigned)(rows * D * 2)),
                    slot, w, toff.k);
    const __amdgpu_buffer_rsrc_t wr =
        make_rsrc(bits + (bh * ntl + t) * (long long)g.nc + rg * kSumRange, (unsigned)(nrange * 8));
#pragma unroll
    for (int k = 0; k < NWI; ++k)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(wr, (lds_ptr_t)(slot + TW + (w * NWI + k) * 128), 4,
                                               (uint32_t)((w * NWI + k) * 256 + lane * 4), 0, 0, 0);
  };
  constexpr int NL = NI + NWI;  // direct-to-LDS loads per wavefront per tile
  // Lane offsets (elements) of the transposed reads of rows 0..15 of a tile
  // (read_tr_one's addresses); rows 16 ks .. add 16 ks D, since the chunk
  // swizzle depends only on the row's low four bits.  Computed once, so the
  // loop holds no address arithmetic.
  uint32_t troff[DT][2];
  {
    const int sl = lane & 15, grp = lane >> 4;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int r = 8 * hf + 4 * h + (sl >> 2);
        const int d = 32 * dt + 16 * (grp & 1) + 4 * (sl & 3);
        troff[dt][h] = (uint32_t)(r * D + (((d >> 3) ^ kt_swz<D>(r)) << 3) + (d & 4));
      }
  }
  issue(0, tl0);
  if (ntau > 1) issue(1, tl1);
  f32x16 acc[NT][DT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) acc[nt][dt] = f32x16{};
  // Step tau (tau % 3 = S) reads slot S and loads tile tau + 2 into slot
  // (S + 2) % 3, which step tau - 1 read.
  auto step = [&](int tau, auto sc) {
    constexpr int S = decltype(sc)::value, SN = (S + 2) % 3;
    uint16_t* slot = S == 0 ? tl0 : (S == 1 ? tl1 : tl2);
    uint16_t* next = SN == 0 ? tl0 : (SN == 1 ? tl1 : tl2);
    // In flight after tile tau: tile tau + 1 (if any), and column stores
    // issued since, which only make this stricter.
    if (tau + 1 < ntau) wait_vmcnt<NL>();
    else wait_vmcnt<0>();
    pipeline_barrier();
    if (tau + 2 < ntau) issue(tau + 2, next);
    uint2 wsel[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
      wsel[nt] = *reinterpret_cast<const uint2*>(slot + TW + 4 * (32 * NT * w + 32 * nt + n));
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      bf16x8 bop[NT];
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        // Cubes 64 t + 16 ks + 8 hf + e, e = 0..7: U = 1 where the bit is
        // clear.  Two bits t2 become one word of two bf16 0/1 values:
        // t2 * 0x8001 puts bit 0 at bit 0 and bit 1 at bit 16, and 0x3F80 is
        // bf16 1.0.
        const uint32_t sel = ((ks < 2) ? wsel[nt].x : wsel[nt].y) >> (16 * (ks & 1) + 8 * hf);
        const uint32_t u = iv[nt] ? ~sel : 0u;
        uint32_t bw[4];
#pragma unroll
        for (int e2 = 0; e2 < 4; ++e2) bw[e2] = ((((u >> (2 * e2)) & 3u) * 0x8001u) & 0x10001u) * 0x3F80u;
        bop[nt] = __builtin_bit_cast(bf16x8, make_uint4(bw[0], bw[1], bw[2], bw[3]));
      }
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        i16x4 part[2];
#pragma unroll
        for (int h = 0; h < 2; ++h)
          part[h] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_ptr)(slot + troff[dt][h] + 16 * ks * D));
        const bf16x8 a =
            __builtin_bit_cast(bf16x8, __builtin_shufflevector(part[0], part[1], 0, 1, 2, 3, 4, 5, 6, 7));
        acc[0][dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bop[0], acc[0][dt], 0, 0, 0);
#pragma unroll
        for (int nt = 1; nt < NT; ++nt)
          if (ntv > nt) acc[nt][dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bop[nt], acc[nt][dt], 0, 0, 0);
      }
    }
    if (tau % ntl == ntl - 1) {
      // Last tile of column xc: its sums out, accumulators cleared.
      const int xc = xc0 + tau / ntl;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        if (iv[nt]) {
          uint16_t* orow = su + (bh * g.nc + ibase + 32 * nt + n) * (long long)(D * D + D) + xc * D;
#pragma unroll
          for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int gq = 0; gq < 4; ++gq) {
              const int d = 32 * dt + 8 * gq + 4 * hf;
              *reinterpret_cast<uint2*>(orow + d) =
                  make_uint2(cvt2(acc[nt][dt][4 * gq], acc[nt][dt][4 * gq + 1]),
                             cvt2(acc[nt][dt][4 * gq + 2], acc[nt][dt][4 * gq + 3]));
            }
        }
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) acc[nt][dt] = f32x16{};
      }
    }
  };
  int tau = 0;
  for (; tau + 3 <= ntau; tau += 3) {
    step(tau, std::integral_constant<int, 0>{});
    step(tau + 1, std::integral_constant<int, 1>{});
    step(tau + 2, std::integral_constant<int, 2>{});
  }
  if (tau < ntau) step(tau, std::integral_constant<int, 0>{});
  if (tau + 1 < ntau) step(tau + 1, std::integral_constant<int, 1>{});
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
  const size_t ntl = ((size_t)g.nc + 63) / 64;
  return ((size_t)g.B * g.H * g.nc * ntl * 8 + 255) / 256 * 256;
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
  uint2* bits = static_cast<uint2*>(ws);
  const int ntl = (g.nc + 63) / 64;
  const long long nrows = (long long)g.B * g.H * g.nc;
  lin_sel_bits<<<dim3((unsigned)((nrows + 255) / 256)), dim3(256), 0, s>>>(idx, topk, bits, g.nc, ntl, nrows);
  // One column tile per wavefront (128 query cubes per workgroup) and runs
  // sized for about three workgroups per compute unit: on the hybrid layer
  // (B = 2, 12 heads, 364 cubes) 0.21 ms against 0.23-0.27 ms for two column
  // tiles per wavefront or other run lengths (one-stream bench, same box).
  const SumPlace pl = make_sum_place<1>(g, 768);
  const dim3 grid((unsigned)(8 * pl.per_xcd));
  if (g.D == 64) hipLaunchKernelGGL((lin_unsel_sum<64, 1>), grid, dim3(kSumThreads), 0, s, st, bits, su, g, pl);
  else hipLaunchKernelGGL((lin_unsel_sum<128, 1>), grid, dim3(kSumThreads), 0, s, st, bits, su, g, pl);
  return hipGetLastError();
}

}  // namespace vsa
