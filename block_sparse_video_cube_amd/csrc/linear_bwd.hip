// Backward of the linear branch: dQ, dK, dV of O_lin = phi(Q) S_U / (phi(Q) . z_U)
// over the unselected cubes U (the SLA/RoLA branch is trained with the sparse
// one: TurboDiffusion article, section "稀疏、蒸馏与全链路量化"; SparkDiffusion
// article, paragraph 3).
//
// For a query row q with w_q = dO_q / den_q and c_q = (dO_q . O_lin_q) / den_q,
// the chain rule through num / den gives, over the key rows r of U(q),
//   d phi(q)  = sum_r (w_q . v_r - c_q) phi(k_r) = S_U w_q - c_q z_U,
//   d phi(k_r) = sum_q (w_q . v_r - c_q) phi(q)   = M_U(r) v_r - m_U(r),
//   dv_r       = sum_q (phi(q) . phi(k_r)) w_q     = M_U(r)^T phi(k_r),
// with M = sum_q phi(q) w_q^T and m = sum_q c_q phi(q) over the query rows
// whose cube left r's cube unselected.  As in the forward, every such sum is
// the total minus the selected blocks, taken block by block on the matrix
// cores:
//   lin_apply (BWD mode)  w, c and phi(Q) per row (recomputes O_lin, den);
//   lin_cube_z            z per key cube, for z_U = z_tot - sum_sel z_j;
//   lin_bwd_state         group partials of M and m, then state_reduce;
//   lin_bwd_dq            per query cube: S_tot w - sum_sel (W V_j^T) phi(K_j)
//                         - c (z_tot - z_sel), times phi'(Q);
//   lin_bwd_dkv           per key cube, over the query cubes that selected it:
//                         dK: M v - m - sum (W_i V^T - c) phi(Q_i), times phi'(K);
//                         dV: M^T phi(K) - sum (phi(Q_i) phi(K)^T) W_i.
#include <math.h>

#include "tile_pipeline.h"

namespace vsa {

namespace {

using namespace tiles;

__device__ __forceinline__ float phi_grad(float x) { return x > 0.f ? 1.f : __expf(x); }

// 64 consecutive floats into LDS, one dword per lane of the calling wavefront.
__device__ __forceinline__ void load_row_f32(const float* src, float* dst, int lane) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(make_rsrc(src, 256), (lds_ptr_t)dst, 4, lane * 4, 0, 0, 0);
}

struct LinBwdWs {
  uint16_t* sd_hi;  // S_tot [d][e], bf16 hi + lo
  uint16_t* sd_lo;
  float* zc;        // z per cube [B, H, Nc, D]
  uint16_t* w;      // [B, H, Np, D]
  float* c;         // [B, H, Np]
  uint16_t* fq;     // [B, H, Np, D]
  uint16_t* md_hi;  // M [d][e]
  uint16_t* md_lo;
  uint16_t* me_hi;  // M^T [e][d]
  uint16_t* me_lo;
  float* m_tot;     // [B, H, D]
  int32_t* cnt;     // transposed block lists
  int32_t* off;
  int32_t* list;
};

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// The forward's linear workspace first, then the backward's own buffers.
LinBwdWs carve_bwd(const KGeom& g, int topk, void* ws, size_t* total) {
  const size_t bh = (size_t)g.B * g.H, D = g.D, Np = g.Np, nc = g.nc;
  size_t off = align256(linear_workspace_bytes(g));
  // Addresses as integers: the sizing call passes no workspace (ws = NULL).
  const uintptr_t base = reinterpret_cast<uintptr_t>(ws);
  auto take = [&](size_t bytes) {
    const uintptr_t p = base + off;
    off += align256(bytes);
    return p;
  };
  LinBwdWs w;
  w.sd_hi = reinterpret_cast<uint16_t*>(take(bh * D * D * 2));
  w.sd_lo = reinterpret_cast<uint16_t*>(take(bh * D * D * 2));
  w.zc = reinterpret_cast<float*>(take(bh * nc * D * 4));
  w.w = reinterpret_cast<uint16_t*>(take(bh * Np * D * 2));
  w.c = reinterpret_cast<float*>(take(bh * Np * 4));
  w.fq = reinterpret_cast<uint16_t*>(take(bh * Np * D * 2));
  w.md_hi = reinterpret_cast<uint16_t*>(take(bh * D * D * 2));
  w.md_lo = reinterpret_cast<uint16_t*>(take(bh * D * D * 2));
  w.me_hi = reinterpret_cast<uint16_t*>(take(bh * D * D * 2));
  w.me_lo = reinterpret_cast<uint16_t*>(take(bh * D * D * 2));
  w.m_tot = reinterpret_cast<float*>(take(bh * D * 4));
  w.cnt = reinterpret_cast<int32_t*>(take(bh * nc * 4));
  w.off = reinterpret_cast<int32_t*>(take(bh * nc * 4));
  w.list = reinterpret_cast<int32_t*>(take(bh * nc * (size_t)topk * 4));
  if (total) *total = off;
  return w;
}

// z_j = sum of the 64 phi(K) rows of cube j (padded rows hold 0).  One
// wavefront per (b, h, cube): lane L sums chunk L % (D/8) of rows L / (D/8),
// + 64/(D/8), ...; the row groups fold with cross-lane exchanges.
template <int D>
__global__ void __launch_bounds__(256) lin_cube_z(const uint16_t* __restrict__ fk, float* __restrict__ zc,
                                                  long long ncubes_total) {
  constexpr int CH = D / 8, RPI = 64 / CH;
  const long long cube = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (cube >= ncubes_total) return;  // whole wavefront
  const int lane = threadIdx.x & 63;
  const uint4* src = reinterpret_cast<const uint4*>(fk + cube * 64 * D);
  float acc[8] = {};
#pragma unroll
  for (int it = 0; it < 64 / RPI; ++it) {
    const uint4 v = src[it * 64 + lane];
    const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      acc[2 * e] += __uint_as_float(w4[e] << 16);
      acc[2 * e + 1] += __uint_as_float(w4[e] & 0xFFFF0000u);
    }
  }
#pragma unroll
  for (int o = CH; o < 64; o *= 2)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] += __shfl_xor(acc[e], o);
  if (lane < CH) {
    float4* dst = reinterpret_cast<float4*>(zc + cube * D + lane * 8);
    dst[0] = make_float4(acc[0], acc[1], acc[2], acc[3]);
    dst[1] = make_float4(acc[4], acc[5], acc[6], acc[7]);
  }
}

// Sum of the group partials of a D x D state (partials [d][e]) and of its
// vector; the state goes out as bf16 hi + lo halves, d-major and/or e-major
// (null outputs are skipped).  One thread per element of one (b, h).
template <int D>
__global__ void __launch_bounds__(256) state_reduce(const float* __restrict__ part, const float* __restrict__ zpart,
                                                    int G, uint16_t* dm_hi, uint16_t* dm_lo, uint16_t* em_hi,
                                                    uint16_t* em_lo, float* zout) {
  const long long bh = blockIdx.y;
  const int f = blockIdx.x * 256 + threadIdx.x;  // d * D + e
  const float* sp = part + bh * G * (long long)D * D;
  float s = 0.f;
#pragma unroll 8
  for (int gi = 0; gi < G; ++gi) s += sp[(long long)gi * D * D + f];
  const int d = f / D, e = f % D;
  const uint16_t hi = f32_to_bf16(s);
  const uint16_t lo = f32_to_bf16(s - bf16_to_f32(hi));
  if (dm_hi) {
    dm_hi[bh * D * D + f] = hi;
    dm_lo[bh * D * D + f] = lo;
  }
  if (em_hi) {
    em_hi[bh * D * D + e * D + d] = hi;
    em_lo[bh * D * D + e * D + d] = lo;
  }
  if (zout && blockIdx.x == gridDim.x - 1 && threadIdx.x < D) {
    float z = 0.f;
    for (int gi = 0; gi < G; ++gi) z += zpart[(bh * G + gi) * D + threadIdx.x];
    zout[bh * D + threadIdx.x] = z;
  }
}

// Group partials of M = sum_q phi(q) w_q^T and m = sum_q c_q phi(q), as
// lin_state does for S and z: per query cube of the group, the phi(Q) and W
// rows go to LDS slots (kt_swz) and both operands are read transposed.
template <int D>
__global__ void __launch_bounds__(256, 2) lin_bwd_state(const uint16_t* __restrict__ fq,
                                                        const uint16_t* __restrict__ wr,
                                                        const float* __restrict__ cr, float* __restrict__ m_part,
                                                        float* __restrict__ mz_part, KGeom g, int gsize, int G) {
  constexpr int CH = D / 8, PT = 64 * CH / 256, RGS = 256 / CH;
  constexpr int NT = (D == 128) ? 4 : 1;
  __shared__ __attribute__((aligned(16))) uint16_t fqs[2][64 * D];
  __shared__ __attribute__((aligned(16))) uint16_t wts[2][64 * D];
  __shared__ float mred[RGS][D];
  const int grp = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, hf = lane >> 5, n = lane & 31;
  const long long bh = (long long)b * g.H + h;
  const int mt = (D == 128) ? w : (w >> 1);
  const int nt0 = (D == 128) ? 0 : (w & 1);
  const int ch = tid % CH;
  const int c0 = grp * gsize, c1 = min(g.nc, c0 + gsize);
  f32x16 acc[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) acc[t] = f32x16{};
  float macc[8] = {};
  uint4 freg[PT], wreg[PT];
  float creg[PT];
  auto load = [&](int c) {
    const long long r0 = bh * g.Np + 64LL * c;
    const uint4* fsrc = reinterpret_cast<const uint4*>(fq + r0 * D);
    const uint4* wsrc = reinterpret_cast<const uint4*>(wr + r0 * D);
#pragma unroll
    for (int p = 0; p < PT; ++p) {
      const int f = tid + 256 * p;
      freg[p] = fsrc[f];
      wreg[p] = wsrc[f];
      creg[p] = cr[r0 + f / CH];
    }
  };
  load(c0);
  for (int c = c0; c < c1; ++c) {
    const int slot = (c - c0) & 1;
#pragma unroll
    for (int p = 0; p < PT; ++p) {
      const int f = tid + 256 * p, row = f / CH;
      const uint32_t fw[4] = {freg[p].x, freg[p].y, freg[p].z, freg[p].w};
#pragma unroll
      for (int e2 = 0; e2 < 4; ++e2) {
        macc[2 * e2] = fmaf(creg[p], __uint_as_float(fw[e2] << 16), macc[2 * e2]);
        macc[2 * e2 + 1] = fmaf(creg[p], __uint_as_float(fw[e2] & 0xFFFF0000u), macc[2 * e2 + 1]);
      }
      const int at = row * D + ((ch ^ kt_swz<D>(row)) << 3);
      *reinterpret_cast<uint4*>(&fqs[slot][at]) = freg[p];
      *reinterpret_cast<uint4*>(&wts[slot][at]) = wreg[p];
    }
    if (c + 1 < c1) load(c + 1);
    pipeline_barrier();  // this cube's slots are complete; the next writes go to the other slot
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const bf16x8 a = read_tr_one<D>(fqs[slot], 16 * kk, mt, lane);
#pragma unroll
      for (int t = 0; t < NT; ++t)
        acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, read_tr_one<D>(wts[slot], 16 * kk, nt0 + t, lane),
                                                         acc[t], 0, 0, 0);
    }
  }
  float* mp = m_part + (bh * G + grp) * (long long)D * D;
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int d = 32 * mt + 8 * (r >> 2) + 4 * hf + (r & 3);
      mp[d * D + 32 * (nt0 + t) + n] = acc[t][r];
    }
#pragma unroll
  for (int e = 0; e < 8; ++e) mred[tid / CH][8 * ch + e] = macc[e];
  __syncthreads();
  if (tid < D) {
    float s = 0.f;
    for (int r = 0; r < RGS; ++r) s += mred[r][tid];
    mz_part[(bh * G + grp) * D + tid] = s;
  }
}

// d phi(Q) and dQ of one query cube.  Wavefront (wq, wk) owns queries
// 32 wq .. +31 and keys 32 wk .. +31 of every selected block, as in the
// forward.  Per block: X^T = V_j W^T (V tile token-major, read as the A
// operand; W in registers as the B operand), rounded to bf16 and negated,
// then d phi(Q)^T += phi(K_j)^T X^T with phi(K_j)^T read transposed.  The
// total S_tot w is split between the key halves (hi on wk = 0, lo on wk = 1).
// Slots are separate LDS objects, so transposed reads of one slot do not
// wait for the loads in flight into the other.
template <int D>
__global__ void __launch_bounds__(kThreads, 2) lin_bwd_dq(const uint16_t* __restrict__ qc,
                                                          const uint16_t* __restrict__ vc,
                                                          const int32_t* __restrict__ idx, int topk,
                                                          const uint16_t* __restrict__ fk,
                                                          const float* __restrict__ z_tot, LinBwdWs t,
                                                          const uint16_t* dq_add, uint16_t* dq, KGeom g,
                                                          Placement pl, int direct) {
  constexpr int DC = D / 16, DT = D / 32;
  __shared__ __attribute__((aligned(16))) uint16_t v0[64 * D];
  __shared__ __attribute__((aligned(16))) uint16_t v1[64 * D];
  __shared__ __attribute__((aligned(16))) uint16_t f0[64 * D];
  __shared__ __attribute__((aligned(16))) uint16_t f1[64 * D];
  __shared__ float zs[D];
  int i, h, b;
  if (!map_workgroup(g, pl, i, h, b)) return;  // whole workgroup leaves before any barrier
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wq = w & 1, wk = w >> 1;
  const int hf = lane >> 5, n = lane & 31;
  const long long bh = (long long)b * g.H + h;
  const int q = 32 * wq + n;
  const long long row = bh * g.Np + 64LL * i + q;
  // idx: the selected cubes, or (direct) the rows of unselected ones, topk long.
  const int32_t* irow = idx + (bh * g.nc + i) * topk;
  const long long hbase = bh * g.Np * D;
  const TileOffsets<D> toff(w, lane);
  const TileOffsets<D, true> ttoff(w, lane);
  constexpr unsigned kTile = 64 * D * 2;
  auto issue = [&](int nb, uint16_t* vs, uint16_t* fs) {
    const long long o = hbase + 64LL * irow[nb] * D;
    issue_k_tile<D>(make_rsrc(vc + o, kTile), vs, w, toff.k);
    issue_k_tile<D>(make_rsrc(fk + o, kTile), fs, w, ttoff.k);
  };
  issue(0, v0, f0);
  bf16x8 wfr[DC];
#pragma unroll
  for (int dc = 0; dc < DC; ++dc) wfr[dc] = *reinterpret_cast<const bf16x8*>(t.w + row * D + 16 * dc + 8 * hf);
  // Total part: this key half's share of S_tot w (rows d, columns q); none
  // in direct mode, where the blocks of U are added instead.
  f32x16 acc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) acc[dt] = f32x16{};
  if (!direct) mat_rows_mfma<D>((wk == 0 ? t.sd_hi : t.sd_lo) + bh * D * D, n, hf, wfr, acc);
  const int prow = pi_row(n);
  const uint32_t xsign = direct ? 0u : 0x80008000u;
  for (int jb = 0; jb < topk; jb += 2) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int nb = jb + u;
      if (nb < topk) {
        uint16_t* vs = u ? v1 : v0;
        uint16_t* fs = u ? f1 : f0;
        wait_vmcnt<0>();
        pipeline_barrier();
        if (nb + 1 < topk) issue(nb + 1, u ? v0 : v1, u ? f0 : f1);
        f32x16 x = f32x16{};
        {
          bf16x8 va[DC];
          read_k<D>(vs, wk, hf, prow, va);
#pragma unroll
          for (int dc = 0; dc < DC; ++dc) x = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[dc], wfr[dc], x, 0, 0, 0);
        }
        uint32_t xw[8];
#pragma unroll
        for (int r = 0; r < 8; ++r) {
          const bf16x2 pk = __builtin_convertvector((f32x2){x[2 * r], x[2 * r + 1]}, bf16x2);
          xw[r] = __builtin_bit_cast(uint32_t, pk) ^ xsign;  // -X (exact in bf16), or +X (direct)
        }
        const bf16x8 xb[2] = {__builtin_bit_cast(bf16x8, make_uint4(xw[0], xw[1], xw[2], xw[3])),
                              __builtin_bit_cast(bf16x8, make_uint4(xw[4], xw[5], xw[6], xw[7]))};
        bf16x8 ta[DT][2];
        read_tr<D>(fs, wk, lane, ta);
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
          for (int kk = 0; kk < 2; ++kk)
            acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ta[dt][kk], xb[kk], acc[dt], 0, 0, 0);
      }
    }
  }

  // Merge the two key halves; then d phi(q) - c_q (z_tot - z_sel), times phi'(q).
  wait_vmcnt<0>();
  __syncthreads();
  float* x = reinterpret_cast<float*>(wq ? v1 : v0);  // DT * 16 * 64 floats: one V slot
  if (wk == 1) {
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) x[(dt * 16 + r) * 64 + lane] = acc[dt][r];
  }
  if (tid < D) {
    // z over the listed cubes, summed in list order; eight loads in flight
    // at a time (no tile load is left to wait for).
    const float* zc = t.zc + bh * g.nc * D + tid;
    float zsum = 0.f;
    int jb = 0;
    for (; jb + 8 <= topk; jb += 8) {
      float zv[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) zv[e] = zc[(long long)irow[jb + e] * D];
#pragma unroll
      for (int e = 0; e < 8; ++e) zsum += zv[e];
    }
    for (; jb < topk; ++jb) zsum += zc[(long long)irow[jb] * D];
    zs[tid] = zsum;
  }
  __syncthreads();
  if (wk == 1) return;
  int ct, cy, cx;
  cube_coords(g, i, ct, cy, cx);
  const bool valid = local_valid(g, ct, cy, cx, q);
  const float cq = t.c[row];
  const float* zt = z_tot + bh * D;
  const uint16_t* qrow = qc + row * D;
  // The addend may alias the output (not restrict): each lane reads its
  // addend elements before it writes the same elements.
  const uint16_t* arow = dq_add ? dq_add + row * D : nullptr;
  uint16_t* out = dq + row * D;
  // Every input of the rows first (one round trip), then the arithmetic.
  uint2 qall[DT][4], aall[DT][4];
  float4 zall[DT][4];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int gq = 0; gq < 4; ++gq) {
      const int d = 32 * dt + 8 * gq + 4 * hf;
      qall[dt][gq] = *reinterpret_cast<const uint2*>(qrow + d);
      aall[dt][gq] = arow ? *reinterpret_cast<const uint2*>(arow + d) : make_uint2(0u, 0u);
      zall[dt][gq] = *reinterpret_cast<const float4*>(zt + d);
    }
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int gq = 0; gq < 4; ++gq) {
      const int d = 32 * dt + 8 * gq + 4 * hf;
      const uint2 qraw = qall[dt][gq];
      const float xq[4] = {__uint_as_float(qraw.x << 16), __uint_as_float(qraw.x & 0xFFFF0000u),
                           __uint_as_float(qraw.y << 16), __uint_as_float(qraw.y & 0xFFFF0000u)};
      const uint2 araw = aall[dt][gq];
      const float ad[4] = {__uint_as_float(araw.x << 16), __uint_as_float(araw.x & 0xFFFF0000u),
                           __uint_as_float(araw.y << 16), __uint_as_float(araw.y & 0xFFFF0000u)};
      const float ztv[4] = {zall[dt][gq].x, zall[dt][gq].y, zall[dt][gq].z, zall[dt][gq].w};
      float o[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int r = 4 * gq + u;
        const float zu = direct ? zs[d + u] : ztv[u] - zs[d + u];  // z over U
        const float dphi = (acc[dt][r] + x[(dt * 16 + r) * 64 + lane]) - cq * zu;
        o[u] = valid ? dphi * phi_grad(xq[u]) + ad[u] : 0.f;
      }
      *reinterpret_cast<uint2*>(out + d) = make_uint2(pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]));
    }
}

// dK (DV = false) or dV (DV = true) of one key cube, over the query cubes that
// selected it.  Wavefront (wk, wq) owns keys 32 wk .. +31 and queries
// 32 wq .. +31; a lane owns a key column, and its V row (dK) or phi(K) row
// (dV) stays in registers as the B operand.  Per query cube i:
//   dK: Y = W_i V^T (W rows in pi order), minus c, negated into bf16, then
//       d phi(K)^T += phi(Q_i)^T (c - Y) with phi(Q_i)^T read transposed;
//   dV: A = phi(Q_i) phi(K)^T, negated into bf16, then dV^T += W_i^T (-A)
//       with W_i^T read transposed.
// The totals M v - m (dK) and M^T phi(K) (dV) are split between the query
// halves (hi on wq = 0, lo on wq = 1; m on wq = 0).
template <int D, bool DV>
__global__ void __launch_bounds__(kThreads, 2) lin_bwd_dkv(const uint16_t* __restrict__ kc,
                                                           const uint16_t* __restrict__ vc,
                                                           const uint16_t* __restrict__ fk, LinBwdWs t, int topk,
                                                           const int32_t* __restrict__ tcnt,
                                                           const int32_t* __restrict__ toffs,
                                                           const int32_t* __restrict__ tlist,
                                                           const uint16_t* add, uint16_t* out, KGeom g,
                                                           Placement pl, int direct) {
  constexpr int DC = D / 16, DT = D / 32;
  __shared__ __attribute__((aligned(16))) uint16_t w0[64 * D];
  __shared__ __attribute__((aligned(16))) uint16_t w1[64 * D];
  __shared__ __attribute__((aligned(16))) uint16_t p0[64 * D];
  __shared__ __attribute__((aligned(16))) uint16_t p1[64 * D];
  __shared__ __attribute__((aligned(16))) float cs[2][64];
  int j, h, b;
  if (!map_workgroup(g, pl, j, h, b)) return;  // whole workgroup leaves before any barrier
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wk = w & 1, wq = w >> 1;
  const int hf = lane >> 5, n = lane & 31;
  const int key = 32 * wk + n;
  const long long bh = (long long)b * g.H + h;
  const long long hbase = bh * g.Np * D, rbase = bh * g.Np;
  const long long krow = rbase + 64LL * j + key;
  const TileOffsets<D, true> toff(w, lane);
  // The transposed lists (t.cnt, t.off, t.list) come as restrict arguments,
  // so that their entries are scalar loads.
  const int cnt = tcnt[bh * g.nc + j];
  const int32_t* list = tlist + bh * (long long)g.nc * topk + toffs[bh * g.nc + j];
  constexpr unsigned kTile = 64 * D * 2;
  auto issue = [&](int m, uint16_t* ws_, uint16_t* ps_, float* cs_) {
    const int i = list[m];
    issue_k_tile<D>(make_rsrc(t.w + hbase + 64LL * i * D, kTile), ws_, w, toff.k);
    issue_k_tile<D>(make_rsrc(t.fq + hbase + 64LL * i * D, kTile), ps_, w, toff.k);
    if (!DV && w == 0) load_row_f32(t.c + rbase + 64LL * i, cs_, lane);
  };
  if (cnt > 0) issue(0, w0, p0, cs[0]);
  // B operand fragments of this lane's key row: V (dK) or phi(K) (dV).
  bf16x8 kb[DC];
  {
    const uint16_t* src = (DV ? fk : vc) + krow * D;
#pragma unroll
    for (int dc = 0; dc < DC; ++dc) kb[dc] = *reinterpret_cast<const bf16x8*>(src + 16 * dc + 8 * hf);
  }
  f32x16 acc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) acc[dt] = f32x16{};
  if (!direct) {
    const uint16_t* mm = (DV ? (wq == 0 ? t.me_hi : t.me_lo) : (wq == 0 ? t.md_hi : t.md_lo)) + bh * D * D;
    mat_rows_mfma<D>(mm, n, hf, kb, acc);
    if (!DV && wq == 0) {
      const float* mt = t.m_tot + bh * D + 4 * hf;
      float4 m4[DT][4];  // all loaded first
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) m4[dt][r4] = *reinterpret_cast<const float4*>(mt + 32 * dt + 8 * r4);
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          acc[dt][4 * r4] -= m4[dt][r4].x;
          acc[dt][4 * r4 + 1] -= m4[dt][r4].y;
          acc[dt][4 * r4 + 2] -= m4[dt][r4].z;
          acc[dt][4 * r4 + 3] -= m4[dt][r4].w;
        }
    }
  }
  const int prow = pi_row(n);
  // Selected query cubes are subtracted from the totals; in direct mode the
  // query cubes that left this key cube unselected are added (sign flipped).
  const uint32_t ysign = direct ? 0x80008000u : 0u;
  // Register r of the 32 x 32 product holds query 32 wq + 16 (r/8) + 8 hf + r%8.
  const int q0 = 32 * wq + 8 * hf;
  for (int mb = 0; mb < cnt; mb += 2) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int m = mb + u;
      if (m < cnt) {
        uint16_t* ws_ = u ? w1 : w0;
        uint16_t* ps_ = u ? p1 : p0;
        wait_vmcnt<0>();
        pipeline_barrier();
        if (m + 1 < cnt) issue(m + 1, u ? w0 : w1, u ? p0 : p1, cs[u ^ 1]);
        f32x16 y = f32x16{};
        {
          bf16x8 ya[DC];
          read_k<D, true>(DV ? ps_ : ws_, wq, hf, prow, ya);
#pragma unroll
          for (int dc = 0; dc < DC; ++dc) y = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ya[dc], kb[dc], y, 0, 0, 0);
        }
        uint32_t yw[8];
        if (!DV) {
          const f32x4* cp = reinterpret_cast<const f32x4*>(&cs[u][0]);
          const f32x4 c4[4] = {cp[q0 / 4], cp[q0 / 4 + 1], cp[(q0 + 16) / 4], cp[(q0 + 16) / 4 + 1]};
#pragma unroll
          for (int r = 0; r < 8; ++r) {
            const int r0 = 2 * r, r1 = 2 * r + 1;
            const f32x2 d2 = {c4[r0 / 4][r0 % 4] - y[r0], c4[r1 / 4][r1 % 4] - y[r1]};
            yw[r] = __builtin_bit_cast(uint32_t, __builtin_convertvector(d2, bf16x2)) ^ ysign;
          }
        } else {
#pragma unroll
          for (int r = 0; r < 8; ++r) {
            const bf16x2 pk = __builtin_convertvector((f32x2){y[2 * r], y[2 * r + 1]}, bf16x2);
            yw[r] = __builtin_bit_cast(uint32_t, pk) ^ 0x80008000u ^ ysign;  // -A (exact in bf16), or +A
          }
        }
        const bf16x8 yb[2] = {__builtin_bit_cast(bf16x8, make_uint4(yw[0], yw[1], yw[2], yw[3])),
                              __builtin_bit_cast(bf16x8, make_uint4(yw[4], yw[5], yw[6], yw[7]))};
        bf16x8 ta[DT][2];
        read_tr<D>(DV ? ws_ : ps_, wq, lane, ta);
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
          for (int kk = 0; kk < 2; ++kk)
            acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ta[dt][kk], yb[kk], acc[dt], 0, 0, 0);
      }
    }
  }

  // Merge the two query halves; dK times phi'(k); padded key rows get none.
  wait_vmcnt<0>();
  __syncthreads();
  float* x = reinterpret_cast<float*>(wk ? w1 : w0);  // DT * 16 * 64 floats: one W slot
  if (wq == 1) {
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) x[(dt * 16 + r) * 64 + lane] = acc[dt][r];
  }
  __syncthreads();
  if (wq == 1) return;
  int ct, cy, cx;
  cube_coords(g, j, ct, cy, cx);
  const bool valid = local_valid(g, ct, cy, cx, key);
  const uint16_t* krw = kc + krow * D;
  // The addend may alias the output (not restrict): each lane reads its
  // addend elements before it writes the same elements.
  const uint16_t* arow = add ? add + krow * D : nullptr;
  uint16_t* orow = out + krow * D;
  // Every input of the rows first (one round trip), then the arithmetic.
  uint2 kall[DT][4], aall[DT][4];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int gq = 0; gq < 4; ++gq) {
      const int d = 32 * dt + 8 * gq + 4 * hf;
      kall[dt][gq] = DV ? make_uint2(0u, 0u) : *reinterpret_cast<const uint2*>(krw + d);
      aall[dt][gq] = arow ? *reinterpret_cast<const uint2*>(arow + d) : make_uint2(0u, 0u);
    }
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int gq = 0; gq < 4; ++gq) {
      const int d = 32 * dt + 8 * gq + 4 * hf;
      float o[4];
      const uint2 kraw = kall[dt][gq];
      const float xk[4] = {__uint_as_float(kraw.x << 16), __uint_as_float(kraw.x & 0xFFFF0000u),
                           __uint_as_float(kraw.y << 16), __uint_as_float(kraw.y & 0xFFFF0000u)};
      const uint2 araw = aall[dt][gq];
      const float ad[4] = {__uint_as_float(araw.x << 16), __uint_as_float(araw.x & 0xFFFF0000u),
                           __uint_as_float(araw.y << 16), __uint_as_float(araw.y & 0xFFFF0000u)};
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int r = 4 * gq + u;
        const float s = acc[dt][r] + x[(dt * 16 + r) * 64 + lane];
        o[u] = valid ? (DV ? s : s * phi_grad(xk[u])) + ad[u] : 0.f;
      }
      *reinterpret_cast<uint2*>(orow + d) = make_uint2(pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]));
    }
}

template <int D>
hipError_t launch_t(const KGeom& g, const uint16_t* qc, const uint16_t* kc, const uint16_t* vc, const uint16_t* vt,
                    const int32_t* idx, int topk, const uint16_t* doc, const float* o_lin, const float* inv_den,
                    const uint16_t* const* add, uint16_t* dq, uint16_t* dk, uint16_t* dv, void* ws, hipStream_t s) {
  hipError_t e = launch_lin_prep(g, kc, vt, ws, s);  // phi(K), S_tot (e-major), z_tot; S partials kept
  if (e != hipSuccess) return e;
  const LinState ls = lin_state_parts(g, ws);
  const LinBwdWs t = carve_bwd(g, topk, ws, nullptr);
  const unsigned bh = (unsigned)(g.B * g.H);
  const long long ncubes = (long long)bh * g.nc;
  // S_tot d-major from the same partials, and z per cube.
  hipLaunchKernelGGL(state_reduce<D>, dim3(D * D / 256, bh), dim3(256), 0, s, ls.s_part, ls.z_part, ls.group_count,
                     t.sd_hi, t.sd_lo, nullptr, nullptr, nullptr);
  hipLaunchKernelGGL(lin_cube_z<D>, dim3((unsigned)((ncubes + 3) / 4)), dim3(256), 0, s, ls.fk, t.zc, ncubes);
  // w, c, phi(Q) per row: from the forward's saved O_lin and 1/den, or recomputed.
  e = launch_lin_bwd_rows(g, qc, vt, idx, topk, o_lin, inv_den, LinBwdRows{doc, t.w, t.c, t.fq}, ws, s);
  if (e != hipSuccess) return e;
  // Direct mode (more than half the cubes selected): the sums run over the
  // unselected cubes (the complement lists the rows pass just built) and
  // over the query cubes that left each key cube unselected, from zero.
  const LinDirect dm = lin_direct(g, topk, ws);
  const int32_t* lists = dm.on ? dm.comp : idx;
  const int len = dm.on ? dm.len : topk;
  if (!dm.on) {
    // M and m (the S partials are consumed: their buffer takes M's partials).
    hipLaunchKernelGGL(lin_bwd_state<D>, dim3(ls.group_count, g.H, g.B), dim3(256), 0, s, t.fq, t.w, t.c,
                       ls.s_part, ls.z_part, g, ls.group_size, ls.group_count);
    hipLaunchKernelGGL(state_reduce<D>, dim3(D * D / 256, bh), dim3(256), 0, s, ls.s_part, ls.z_part,
                       ls.group_count, t.md_hi, t.md_lo, t.me_hi, t.me_lo, t.m_tot);
  }
  e = launch_block_lists_t(g, lists, len, t.cnt, t.off, t.list, s);
  if (e != hipSuccess) return e;
  const Placement pl = make_placement(g);
  hipLaunchKernelGGL(lin_bwd_dq<D>, dim3(grid_size(g)), dim3(kThreads), 0, s, qc, vc, lists, len, ls.fk, ls.z_tot, t,
                     add[0], dq, g, pl, dm.on);
  hipLaunchKernelGGL((lin_bwd_dkv<D, false>), dim3(grid_size(g)), dim3(kThreads), 0, s, kc, vc, ls.fk, t, len,
                     t.cnt, t.off, t.list, add[1], dk, g, pl, dm.on);
  hipLaunchKernelGGL((lin_bwd_dkv<D, true>), dim3(grid_size(g)), dim3(kThreads), 0, s, kc, vc, ls.fk, t, len,
                     t.cnt, t.off, t.list, add[2], dv, g, pl, dm.on);
  return hipGetLastError();
}

}  // namespace

size_t linear_bwd_workspace_bytes(const KGeom& g, int topk) {
  size_t total = 0;
  carve_bwd(g, topk, nullptr, &total);
  return total;
}

hipError_t launch_linear_bwd(const KGeom& g, const uint16_t* qc, const uint16_t* kc, const uint16_t* vc,
                             const uint16_t* vt, const int32_t* idx, int topk, const uint16_t* doc,
                             const float* o_lin, const float* inv_den, const uint16_t* dq_add,
                             const uint16_t* dk_add, const uint16_t* dv_add, uint16_t* dq, uint16_t* dk, uint16_t* dv,
                             void* ws, hipStream_t s) {
  const uint16_t* const add[3] = {dq_add, dk_add, dv_add};
  if (g.D == 64) return launch_t<64>(g, qc, kc, vc, vt, idx, topk, doc, o_lin, inv_den, add, dq, dk, dv, ws, s);
  return launch_t<128>(g, qc, kc, vc, vt, idx, topk, doc, o_lin, inv_den, add, dq, dk, dv, ws, s);
}

}  // namespace vsa
