// Tile pipeline shared by the block-sparse streaming kernels (fine stage and
// linear-branch correction): gfx950 MFMA operand layouts, LDS swizzles and
// the direct buffer->LDS loads of 64-row cube tiles.
//
// Operand conventions (v_mfma_f32_32x32x16_bf16, per wavefront):
//  * A tile of K (64 keys x D, token-major) is read as the A operand of
//    S^T = K Q^T; Q (or phi(Q)) stays in registers as the B operand.
//  * A tile of V^T (D x 64 keys, i.e. the cube stored transposed) is read as
//    the A operand of O^T += V^T P^T; P is the S^T accumulator itself.
#pragma once

#include "common.h"

namespace vsa {
namespace tiles {

constexpr int kThreads = 256;  // four wavefronts per query cube

// A compile-time step index (a ring slot is a function of it), passed to
// generic lambdas that run one pipeline step.
template <int N>
struct StepC {
  static constexpr int value = N;
};

// Wait until at most N vector-memory loads of this wavefront are in flight
// (s_waitcnt vmcnt(N), gfx9 encoding: vmcnt in bits 3:0 and 15:14, the other
// counters left at their maximum).  Loads complete in issue order, so this
// waits for every direct-to-LDS tile load except the N most recent ones.  The
// workgroup fence of __syncthreads() treats those loads as loads and does not
// wait for them by itself.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt field");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}

// Workgroup barrier of the tile pipeline.  Every wavefront has already waited
// (wait_vmcnt) for its share of the tiles that the next step reads, so after
// the barrier those tiles are complete in LDS; its own LDS reads have
// completed (lgkmcnt(0)), so the buffers the next loads overwrite are free.
// A plain s_barrier is used instead of __syncthreads(): the release fence of
// the latter would also wait for the tile loads still in flight.
__device__ __forceinline__ void pipeline_barrier() {
  asm volatile("" ::: "memory");  // keep the compiler's LDS accesses on their side
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

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

// Token-major tiles that are also read transposed (read_tr) use another chunk
// swizzle: at D = 128 the two 2-bit fields of the row index trade places, so
// the four rows that one 16-lane group of a transposed read touches land in
// four different quarters of the banks; read_k stays conflict-free (the map
// is a bijection of row % 16).  At D = 64 two rows share 256 bytes and the
// same idea takes (row >> 1) & 1 to the top bit.
template <int D>
__device__ __forceinline__ int kt_swz(int row) {
  return (D == 128) ? (((row & 3) << 2) | ((row >> 2) & 3)) : ((((row >> 1) & 1) << 2) | ((row >> 2) & 3));
}
template <int D, bool TR>
__device__ __forceinline__ int row_swz(int row) {
  return TR ? kt_swz<D>(row) : k_swz<D>(row);
}

// Per-lane byte offsets of this wave's share of one K tile and one V^T tile.
// Every buffer_load_dwordx4 ... lds writes 64 consecutive 16-byte LDS slots;
// lane L fills slot L with the global chunk that the swizzle maps there.
// TR: K-style tiles in the kt_swz layout.
template <int D, bool TR = false>
struct TileOffsets {
  static constexpr int KRPI = 512 / D;  // K rows per 1 KB instruction
  static constexpr int NI = D / 32;     // instructions per wave per tile
  uint32_t k[NI], v[NI];
  __device__ __forceinline__ TileOffsets(int w, int lane) {
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int row = (w * NI + i) * KRPI + lane / (D / 8);
      k[i] = (uint32_t)(row * D + ((lane % (D / 8)) ^ row_swz<D, TR>(row)) * 8) * 2u;
      const int vrow = (w * NI + i) * 8 + (lane >> 3);
      v[i] = (uint32_t)(vrow * 64 + ((lane & 7) ^ v_swz(vrow)) * 8) * 2u;
    }
  }
};

// Issue the direct-to-LDS loads of one K tile or one V^T tile (this wave's
// share).  The buffer resource covers exactly one tile, so every load is
// range-checked by the hardware.
template <int D>
__device__ __forceinline__ void load_k_tile(const uint16_t* ktile, uint16_t* klds, int w, const TileOffsets<D>& off) {
  constexpr int KRPI = TileOffsets<D>::KRPI, NI = TileOffsets<D>::NI;
  const __amdgpu_buffer_rsrc_t kr = make_rsrc(ktile, 64 * D * 2);
#pragma unroll
  for (int i = 0; i < NI; ++i)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(kr, (lds_ptr_t)(klds + (w * NI + i) * KRPI * D), 16, off.k[i], 0, 0, 0);
}

template <int D>
__device__ __forceinline__ void load_v_tile(const uint16_t* vtile, uint16_t* vlds, int w, const TileOffsets<D>& off) {
  constexpr int NI = TileOffsets<D>::NI;
  const __amdgpu_buffer_rsrc_t vr = make_rsrc(vtile, 64 * D * 2);
#pragma unroll
  for (int i = 0; i < NI; ++i)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(vr, (lds_ptr_t)(vlds + (w * NI + i) * 8 * 64), 16, off.v[i], 0, 0, 0);
}

// The same loads from a buffer resource built by the caller and this wave's
// lane offsets (TileOffsets::k or ::v).  Kernels whose tiles change every
// step use these.
template <int D>
__device__ __forceinline__ void issue_k_tile(__amdgpu_buffer_rsrc_t kr, uint16_t* klds, int w, const uint32_t* off) {
  constexpr int NI = D / 32, KRPI = 512 / D;
#pragma unroll
  for (int e = 0; e < NI; ++e)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(kr, (lds_ptr_t)(klds + (w * NI + e) * KRPI * D), 16, off[e], 0, 0, 0);
}

template <int D>
__device__ __forceinline__ void issue_v_tile(__amdgpu_buffer_rsrc_t vr, uint16_t* vlds, int w, const uint32_t* off) {
  constexpr int NI = D / 32;
#pragma unroll
  for (int e = 0; e < NI; ++e)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(vr, (lds_ptr_t)(vlds + (w * NI + e) * 8 * 64), 16, off[e], 0, 0, 0);
}

// acc[dt] += (rows 32 dt .. +31 of a row-major D x D bf16 matrix M) . B,
// on the matrix cores: lane (hf, n) reads row 32 dt + n, elements
// 16 dc + 8 hf .. +7 as A operands; b holds the B fragments.  Row block
// dt + 1 is loaded while block dt is multiplied, so the 16 KB per wavefront
// arrive in two round trips instead of one per load.
template <int D>
__device__ __forceinline__ void mat_rows_mfma(const uint16_t* m, int n, int hf, const bf16x8 (&b)[D / 16],
                                              f32x16 (&acc)[D / 32]) {
  constexpr int DC = D / 16, DT = D / 32;
  const uint16_t* src = m + n * D + 8 * hf;
  bf16x8 a[2][DC];
#pragma unroll
  for (int dc = 0; dc < DC; ++dc) a[0][dc] = *reinterpret_cast<const bf16x8*>(src + 16 * dc);
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) {
    if (dt + 1 < DT) {
#pragma unroll
      for (int dc = 0; dc < DC; ++dc)
        a[(dt + 1) & 1][dc] = *reinterpret_cast<const bf16x8*>(src + 32 * (dt + 1) * D + 16 * dc);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int dc = 0; dc < DC; ++dc)
      acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[dt & 1][dc], b[dc], acc[dt], 0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Gathering a token-major tile straight from raster-order rows
// ([B, S, heads, D]: consecutive tokens of one head are heads * D elements
// apart).  Local token l of a cube sits (lt * Hg + ly) * W + lx tokens after
// the cube's first token, (lt, ly, lx) = (l / 16, l / 4 % 4, l % 4), so each
// lane's offset within a cube is fixed; only the buffer base moves from cube
// to cube.  raster_lane_offsets: this wave's lanes, for instructions
// e < D / 32 of a tile load, the byte offset of its (swizzled) 16-byte chunk
// and the local token index of its row.
template <int D>
__device__ __forceinline__ void raster_lane_offsets(const KGeom& g, int w, int lane, uint32_t* off, int* row) {
  constexpr int NI = D / 32, KRPI = 512 / D;
#pragma unroll
  for (int e = 0; e < NI; ++e) {
    const int r = (w * NI + e) * KRPI + lane / (D / 8);
    const int rowoff = ((r >> 4) * g.Hg + ((r >> 2) & 3)) * g.W + (r & 3);
    off[e] = (uint32_t)(rowoff * g.H * D + ((lane % (D / 8)) ^ k_swz<D>(r)) * 8) * 2u;
    row[e] = r;
  }
}

// Buffer resource over the raster rows from the first token of cube j to the
// end of the head's tokens (xhead: element (b, token 0, h, 0)), and the lane
// offsets for it.  Padded tokens of a partial cube get an offset past the
// range, so the hardware range check returns zeros for them.
template <int D, bool PARTIAL>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t raster_tile(const uint16_t* xhead, const KGeom& g, int j,
                                                             const uint32_t* off, const int* row, uint32_t* out) {
  constexpr int NI = D / 32;
  int ct, cy, cx;
  cube_coords(g, j, ct, cy, cx);
  const long long corner = ((long long)(4 * ct) * g.Hg + 4 * cy) * g.W + 4 * cx;
  const long long pitch = (long long)g.H * D;
#pragma unroll
  for (int e = 0; e < NI; ++e) out[e] = off[e];
  if (PARTIAL) {
    const int nt = g.T - 4 * ct, ny = g.Hg - 4 * cy, nx = g.W - 4 * cx;
#pragma unroll
    for (int e = 0; e < NI; ++e) {
      const int r = row[e];
      const bool ok = (r >> 4) < nt && ((r >> 2) & 3) < ny && (r & 3) < nx;
      out[e] = ok ? off[e] : 0xFFFFFFF0u;
    }
  }
  return make_rsrc(xhead + corner * pitch, (unsigned)((g.S - corner) * pitch * 2));
}

// K fragments of S^T = K Q^T for this wave's key half (rows in pi order).
template <int D, bool TR = false>
__device__ __forceinline__ void read_k(const uint16_t* klds, int wk, int hf, int prow, bf16x8 (&ka)[D / 16]) {
  const int krow = 32 * wk + prow;
#pragma unroll
  for (int dc = 0; dc < D / 16; ++dc)
    ka[dc] = *reinterpret_cast<const bf16x8*>(klds + krow * D + (((2 * dc + hf) ^ row_swz<D, TR>(krow)) * 8));
}

// The transpose of a token-major tile (kt_swz layout) as A operands:
// xa[dt][kk] of lane (hf, n) holds X[32 w + 16 kk + 8 hf + e][32 dt + n],
// e = 0..7, the same fragments read_v gives from a stored transpose.
// ds_read_b64_tr_b16 works on groups of 16 lanes: each lane points at 4
// consecutive elements of one row, and lane l of the group receives element
// l % 4 of the rows pointed at by lanes l / 4, 4 + l / 4, 8 + l / 4 and
// 12 + l / 4.  So lane s of the group points at row (s / 4) of a 4-row
// slice, columns 4 (s % 4) .. +3 of a 16-column slice, and lane l gets
// column l of the 4 rows.  Two reads give the 8 rows of one fragment.
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4* lds_i16x4_ptr;
// One such fragment: rows row0 + 8 hf + e (row0 a multiple of 16), column
// 32 dt + n.
template <int D>
__device__ __forceinline__ bf16x8 read_tr_one(const uint16_t* lds, int row0, int dt, int lane) {
  const int s = lane & 15, grp = lane >> 4, hf = grp >> 1;
  i16x4 part[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int r = row0 + 8 * hf + 4 * h + (s >> 2);
    const int d = 32 * dt + 16 * (grp & 1) + 4 * (s & 3);
    const uint16_t* p = lds + r * D + (((d >> 3) ^ kt_swz<D>(r)) << 3) + (d & 4);
    part[h] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_ptr)(p));
  }
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(part[0], part[1], 0, 1, 2, 3, 4, 5, 6, 7));
}

template <int D>
__device__ __forceinline__ void read_tr(const uint16_t* lds, int w, int lane, bf16x8 (&xa)[D / 32][2]) {
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) xa[dt][kk] = read_tr_one<D>(lds, 32 * w + 16 * kk, dt, lane);
}

// V^T fragments of O^T += V^T P^T for this wave's 32 keys (2 chunks of 16).
template <int D>
__device__ __forceinline__ void read_v(const uint16_t* vlds, int wk, int hf, int n, bf16x8 (&va)[D / 32][2]) {
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) {
    const int vrow = 32 * dt + n;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const int chunk = 4 * wk + 2 * kk + hf;
      va[dt][kk] = *reinterpret_cast<const bf16x8*>(vlds + vrow * 64 + ((chunk ^ v_swz(vrow)) * 8));
    }
  }
}

// Packed tiles.  A tile's 64 key rows are four slots of 16 rows; slot s
// holds rows 16 sc .. 16 sc + 15 of key cube j in compact order (the cube's
// valid keys first), of which the first `count` are valid keys.  A slot code
// is j << 8 | sc << 5 | count, and 0 for an empty slot.  Wavefront w loads
// slot w of K (rows 16 w .. 16 w + 15 of the tile, in the TileOffsets layout)
// and of V, whose slots are stored channel-major in HBM ([4][D][16] per cube)
// and in LDS, so each is one contiguous D x 16 block.
__device__ __forceinline__ int slot_cube(int code) { return code >> 8; }
__device__ __forceinline__ int slot_sub(int code) { return (code >> 5) & 3; }
__device__ __forceinline__ int slot_count(int code) { return code & 31; }

// Buffer resource for wavefront w's share of the K tile (slot w): based so
// that the TileOffsets lane offsets of rows 16 w .. 16 w + 15 land on the
// slot's rows; only the slot's `count` valid rows are in range (the rest
// read as zero without a memory access).
template <int D>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t k_slot_rsrc(const uint16_t* khead, int code, int w) {
  const int cnt = slot_count(code);
  const long long row0 = 64LL * slot_cube(code) + 16 * slot_sub(code) - 16 * w;
  return make_rsrc(khead + row0 * D, cnt ? (unsigned)((16 * w + cnt) * D * 2) : 0u);
}

// Buffer resource of one V slot (D x 16, 16 * D * 2 contiguous bytes).
template <int D>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t v_slot_rsrc(const uint16_t* vhead, int code) {
  const long long off = (64LL * slot_cube(code) + 16 * slot_sub(code)) * D;
  return make_rsrc(vhead + off, slot_count(code) ? (unsigned)(16 * D * 2) : 0u);
}

// In LDS a V slot is D channel rows of two 16-byte halves (keys 0..7 and
// 8..15); the halves of rows with bit 3 set trade places, so the 16 lanes of
// one pass of a 16-byte read (16 consecutive rows, one half) cover all banks.
__device__ __forceinline__ int v_slot_half(int row, int h) { return h ^ ((row >> 3) & 1); }

// Lane offsets of this wavefront's V slot load: lane L of instruction e fills
// 16-byte position p = 64 e + L of the slot (row p / 2, half p % 2 after the
// swap), from the same row and logical half of the slot in HBM.
template <int D>
__device__ __forceinline__ void v_slot_offsets(int lane, uint32_t* off) {
#pragma unroll
  for (int e = 0; e < D / 32; ++e) {
    const int p = 64 * e + lane, row = p >> 1;
    off[e] = (uint32_t)(2 * row + v_slot_half(row, p & 1)) * 16u;
  }
}

// V^T fragments from a slot-layout V tile in LDS: the same operands as
// read_v (chunk 4 wk + 2 kk + hf of channel row 32 dt + n is keys 8 hf ..
// 8 hf + 7 of slot 2 wk + kk).
template <int D>
__device__ __forceinline__ void read_v_slots(const uint16_t* vlds, int wk, int hf, int n,
                                             bf16x8 (&va)[D / 32][2]) {
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) {
    const int row = 32 * dt + n;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
      va[dt][kk] = *reinterpret_cast<const bf16x8*>(vlds + (2 * wk + kk) * (D * 16) + row * 16 +
                                                    8 * v_slot_half(row, hf));
  }
}

// Keys of a packed tile past their slot's count take no weight.  In the S^T
// accumulator, register r of lane half hf holds position 8 hf + r % 8 of slot
// 2 wk + r / 8; c0, c1 are the counts of this wavefront's two slots.
__device__ __forceinline__ void mask_slots(f32x16& s, int c0, int c1, int hf) {
  const int l0 = c0 - 8 * hf, l1 = c1 - 8 * hf;
#pragma unroll
  for (int r = 0; r < 16; ++r) s[r] = ((r & 7) < (r < 8 ? l0 : l1)) ? s[r] : -INFINITY;
}

// Padded keys of key cube j take no weight: their logits become -inf.
// In an S^T = K Q^T tile (keys in rows, read in pi order) accumulator
// register r of lane half hf holds local key 32 wk + 16 (r/8) + 8 hf + r%8,
// i.e. local (t, y, x) = (2 wk + r/8, 2 hf + (r%8)/4, r%4): the t and x tests
// are the same for the whole wavefront, the y test depends on the lane half
// only.  Branch-free, so it can sit inside an interleaved region.
__device__ __forceinline__ void mask_keys(f32x16& s, const KGeom& g, int j, int wk, int hf) {
  int ct, cy, cx;
  cube_coords(g, j, ct, cy, cx);
  const int nt = g.T - 4 * ct, ny = g.Hg - 4 * cy, nx = g.W - 4 * cx;
  const bool y0 = 2 * hf < ny, y1 = 2 * hf + 1 < ny;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const bool tx = (2 * wk + (r >> 3) < nt) && ((r & 3) < nx);
    const bool ok = tx && (((r >> 2) & 1) ? y1 : y0);
    s[r] = ok ? s[r] : -INFINITY;
  }
}

// XCD-aware placement.  Workgroups are handed to the 8 XCDs round-robin, so
// XCD x receives ids x, x+8, x+16, ...  Every workgroup visits its selected
// key cubes in ascending order and all carry the same work, so workgroups
// that run together sweep the key range together and share the tiles in
// their XCD's L2 while they pass.  To keep the workgroups that run together
// on one XCD inside a single head, each (b, h) is cut into `splits` ranges
// of consecutive query cubes (the fewest that make the number of ranges a
// multiple of 8, so the XCDs stay balanced), and XCD x takes ranges
// x, x+8, ... one after the other.
struct Placement {
  int splits;      // query-cube ranges per (b, h)
  int range_len;   // query cubes per range
  int ranges;      // B * H * splits
  int per_xcd;     // ranges per XCD
};

inline Placement make_placement(const KGeom& g) {
  Placement p;
  const int bh = g.B * g.H;
  int s = 1;
  while ((bh * s) % 8 != 0 && s < 8 && (g.nc + s) / (s + 1) >= 64) ++s;
  p.splits = s;
  p.range_len = (g.nc + s - 1) / s;
  p.ranges = bh * s;
  p.per_xcd = (p.ranges + 7) / 8;
  return p;
}

inline unsigned grid_size(const KGeom& g) {
  const Placement p = make_placement(g);
  return (unsigned)(8 * p.per_xcd * p.range_len);
}

// Query cube i and head (h, b) of this workgroup; false for the ids past the
// end (the whole workgroup then leaves before any barrier).
__device__ __forceinline__ bool map_workgroup(const KGeom& g, const Placement& p, int& i, int& h, int& b) {
  const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
  const int rk = slot / p.range_len;          // k-th range of this XCD
  const int range = xcd + 8 * rk;             // global range index
  if (range >= p.ranges) return false;
  const int bhi = range / p.splits, sp = range - bhi * p.splits;
  i = sp * p.range_len + (slot - rk * p.range_len);
  h = bhi % g.H;
  b = bhi / g.H;
  return i < g.nc;
}

}  // namespace tiles
}  // namespace vsa
