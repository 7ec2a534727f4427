// Device-side definitions shared by the gfx950 kernels: the geometry they take by value,
// vector types, cube indexing and bf16 helpers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace vsa {

// Geometry handed to every kernel by value.
struct KGeom {
  int B, H, D;       // batch, heads, head_dim
  int T, Hg, W;      // valid latent grid
  int ct, ch, cw;    // cubes per axis
  int nc;            // cubes
  long long S;       // tokens
  long long Np;      // cube-major rows = 64 * nc
  int partial;       // 1 if some cube holds padded tokens
};

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Cube coordinates of cube c.
__device__ __forceinline__ void cube_coords(const KGeom& g, int c, int& ct, int& cy, int& cx) {
  cx = c % g.cw;
  const int r = c / g.cw;
  cy = r % g.ch;
  ct = r / g.ch;
}

// Is local token l of the cube at (ct, cy, cx) inside the valid grid?
__device__ __forceinline__ bool local_valid(const KGeom& g, int ct, int cy, int cx, int l) {
  return (4 * ct + (l >> 4)) < g.T && (4 * cy + ((l >> 2) & 3)) < g.Hg && (4 * cx + (l & 3)) < g.W;
}

// Are all 64 tokens of the cube valid?
__device__ __forceinline__ bool cube_full(const KGeom& g, int ct, int cy, int cx) {
  return 4 * ct + 3 < g.T && 4 * cy + 3 < g.Hg && 4 * cx + 3 < g.W;
}

// Number of valid tokens of a cube.
__device__ __forceinline__ int cube_count(const KGeom& g, int ct, int cy, int cx) {
  const int nt = min(4, g.T - 4 * ct), ny = min(4, g.Hg - 4 * cy), nx = min(4, g.W - 4 * cx);
  return nt * ny * nx;
}

// Row of local token l inside its cube in compact order: the cube's valid
// tokens first, in raster order within the cube (rank among them), then its
// padded slots in the same order.  A bijection of 0..63; the identity for a
// full cube.
__device__ __forceinline__ int compact_row(const KGeom& g, int ct, int cy, int cx, int l) {
  const int nt = min(4, g.T - 4 * ct), ny = min(4, g.Hg - 4 * cy), nx = min(4, g.W - 4 * cx);
  const int lt = l >> 4, ly = (l >> 2) & 3, lx = l & 3;
  const bool in_t = lt < nt, in_y = ly < ny;
  const int before = min(lt, nt) * ny * nx + (in_t ? min(ly, ny) * nx + (in_y ? min(lx, nx) : 0) : 0);
  const bool valid = in_t && in_y && lx < nx;
  return valid ? before : nt * ny * nx + (l - before);
}

// Buffer resource over `bytes` bytes at `base` (raw, unswizzled, dword data
// format): loads outside the range return zero instead of faulting.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, unsigned bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

typedef __attribute__((address_space(3))) void* lds_ptr_t;

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(((uint32_t)b) << 16);
}

// fp32 -> bf16 bits, round to nearest even (inputs here are finite).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  const uint32_t u = __float_as_uint(f);
  return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return (uint32_t)f32_to_bf16(lo) | ((uint32_t)f32_to_bf16(hi) << 16);
}

// Feature map of the linear branch: phi(x) = elu(x) + 1 (alpha = 1).
__device__ __forceinline__ float phi_elu1(float x) { return x > 0.f ? x + 1.f : __expf(x); }

// phi of the two bf16 values packed in w (low half first), rounded to bf16
// by one v_cvt_pk_bf16_f32 (round to nearest even, as f32_to_bf16 for the
// finite values here).
__device__ __forceinline__ uint32_t phi2_bf16(uint32_t w) {
  const f32x2 x = {phi_elu1(__uint_as_float(w << 16)), phi_elu1(__uint_as_float(w & 0xFFFF0000u))};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(x, bf16x2));
}

}  // namespace vsa
