// Shared definitions of the gfx950 kernels (device side) and their host launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "vsa_cube.h"

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

KGeom make_kgeom(const vsa_geom& g, const vsa_dims& d);

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

// Host launchers (each returns hipSuccess or the launch error).
namespace vsa {
hipError_t launch_permute(const KGeom& g, const uint16_t* x, uint16_t* xc, int layout, hipStream_t s);
hipError_t launch_permute_pool(const KGeom& g, const uint16_t* x, uint16_t* xc, float* mean, bool compact,
                               hipStream_t s);
hipError_t launch_unpermute(const KGeom& g, const uint16_t* xc, uint16_t* x, hipStream_t s);
hipError_t launch_select(const KGeom& g, const uint16_t* qc, const uint16_t* kc, int topk, int32_t* idx,
                         void* ws, hipStream_t s);
size_t select_workspace_bytes(const KGeom& g);
hipError_t launch_select_pooled(const KGeom& g, const float* qbar, const float* kbar, int topk, int32_t* idx,
                                float* scores, hipStream_t s);
size_t select_pooled_workspace_bytes(const KGeom& g);
hipError_t launch_attn_fwd(const KGeom& g, const uint16_t* qc, const uint16_t* kc, const uint16_t* vt,
                           const int32_t* idx, int topk, float scale, uint16_t* oc, float* oc_f32, float* lse,
                           hipStream_t s);
// o: raster bf16 output (may be null when o_f32 is given); o_f32: optional
// fp32 output in cube-major rows.
hipError_t launch_attn_fwd_raster(const KGeom& g, const uint16_t* q, const uint16_t* k, bool k_raster,
                                  const uint16_t* vt, const int32_t* idx, int topk, float scale, uint16_t* o,
                                  float* o_f32, float* lse, hipStream_t s);
// Packed fine stage: K in compact cube-major rows, V in the slot layout;
// q/o raster (raster = true) or cube-major.  ws: the packing plan of a grid
// with partial cubes (attn_packed_workspace_bytes; 0 for full grids).
size_t attn_packed_workspace_bytes(const KGeom& g, int topk);
hipError_t launch_attn_fwd_packed(const KGeom& g, const uint16_t* q, bool raster, const uint16_t* kc,
                                  const uint16_t* vs, const int32_t* idx, int topk, float scale, uint16_t* o,
                                  float* lse, void* ws, hipStream_t s);
// The packing plan and launch order of a grid with partial cubes into ws (the
// packed stages' workspace; nothing for a full grid).
hipError_t launch_packed_plan(const KGeom& g, const int32_t* idx, int topk, void* ws, hipStream_t s);
// o_lin, inv_den: optional (both or neither) fp32 copies of O_lin [B, H, Np, D]
// and of 1/den [B, H, Np] for the backward.
// raster: q and the output oc are raster [B, S, H, D] (padded query rows not
// written) instead of cube-major rows; o_sparse, o_lin and inv_den stay
// cube-major.
hipError_t launch_linear(const KGeom& g, const uint16_t* qc, const uint16_t* kc, const uint16_t* vt,
                         const int32_t* idx, int topk, const float* o_sparse, uint16_t* oc, float* o_lin,
                         float* inv_den, bool raster, void* ws, hipStream_t s);
// launch_linear without the state pass: ws must hold phi(K), S_tot and z_tot
// from launch_lin_prep (write_fk) for the same keys and values.
hipError_t launch_linear_apply(const KGeom& g, const uint16_t* qc, const uint16_t* vt, const int32_t* idx, int topk,
                               const float* o_sparse, uint16_t* oc, float* o_lin, float* inv_den, bool raster,
                               void* ws, hipStream_t s);
size_t linear_workspace_bytes(const KGeom& g);
// The parts of the linear workspace the selected-block correction reads:
// phi(K) token-major bf16 [B, H, Np, D], S_tot^T as bf16 hi + lo [B, H, D, D],
// z_tot fp32 [B, H, D].  launch_lin_prep fills them (lin_state, lin_reduce).
struct LinTensors {
  const uint16_t* fk;
  const uint16_t* st_hi;
  const uint16_t* st_lo;
  const float* z_tot;
};
LinTensors lin_tensors(const KGeom& g, void* ws);
// Per-row inputs of the linear branch's backward, written by the forward's
// selected-block pass in its backward mode (all token-major [B, H, Np, ...]).
struct LinBwdRows {
  const uint16_t* doc;  // dO, bf16
  uint16_t* w;          // dO / den, bf16
  float* c;             // (dO . O_lin) / den, fp32 [B, H, Np]
  uint16_t* fq;         // phi(Q), bf16
};
// With the forward's saved O_lin and 1/den (both non-null) the rows come from
// them (lin_rows); otherwise the selected-block pass recomputes them.
hipError_t launch_lin_bwd_rows(const KGeom& g, const uint16_t* qc, const uint16_t* vt, const int32_t* idx, int topk,
                               const float* o_lin, const float* inv_den, const LinBwdRows& br, void* ws,
                               hipStream_t s);
// The parts of the linear workspace the backward reuses: phi(K), the group
// partials of the state (reused for the backward's own state), z_tot.
struct LinState {
  const uint16_t* fk;
  float* s_part;  // [B, H, count, D, D]
  float* z_part;  // [B, H, count, D]
  const float* z_tot;
  int group_size, group_count;
};
LinState lin_state_parts(const KGeom& g, void* ws);
// Direct mode of the linear branch (more than half the cubes selected): the
// complement lists in the workspace ([B, H, Nc, len] int32, ascending), built
// by the forward's selected-block pass (launch_linear, launch_lin_bwd_rows).
struct LinDirect {
  int on;
  const int32_t* comp;
  int len;  // Nc - topk
};
LinDirect lin_direct(const KGeom& g, int topk, void* ws);
hipError_t launch_block_lists_t(const KGeom& g, const int32_t* idx, int topk, int32_t* cnt, int32_t* off,
                                int32_t* list, hipStream_t s);
size_t linear_bwd_workspace_bytes(const KGeom& g, int topk);
hipError_t launch_linear_bwd(const KGeom& g, const uint16_t* qc, const uint16_t* kc, const uint16_t* vc,
                             const uint16_t* vt, const int32_t* idx, int topk, const uint16_t* doc,
                             const float* o_lin, const float* inv_den, const uint16_t* dq_add,
                             const uint16_t* dk_add, const uint16_t* dv_add, uint16_t* dq, uint16_t* dk, uint16_t* dv,
                             void* ws, hipStream_t s);
// write_fk = false: the totals only (S_tot, z_tot), no phi(K) rows.
hipError_t launch_lin_prep(const KGeom& g, const uint16_t* kc, const uint16_t* vt, void* ws, hipStream_t s,
                           bool write_fk = true);
hipError_t launch_attn_lin_fwd(const KGeom& g, const uint16_t* qc, const uint16_t* kc, const uint16_t* vt,
                               const int32_t* idx, int topk, float scale, void* ws, uint16_t* oc, float* lse,
                               hipStream_t s);
hipError_t launch_sta_index(const KGeom& g, int wt, int wh, int ww, int32_t* idx, hipStream_t s);
size_t attn_bwd_workspace_bytes(const KGeom& g, int topk);
hipError_t launch_mfma_probe(int blocks, int iters, float* sink, unsigned long long* clk, hipStream_t s);
hipError_t launch_hbm_probe(int kind, const void* src, void* dst, long long words, hipStream_t s);
size_t quant_workspace_bytes(const KGeom& g);
hipError_t launch_quant(const KGeom& g, const uint16_t* q, const uint16_t* k, const uint16_t* v, uint8_t* q8,
                        float* qs, uint8_t* k8, float* ks, uint8_t* v8t, float* vs, float* qmean, float* kmean,
                        void* ws, hipStream_t s, bool packed = false);
// The device address of the quantizer's static scratch array (VSA_QUANT_SCRATCH_WORDS
// words) on the device of stream s, looked up once per device.
hipError_t quant_scratch(hipStream_t s, uint32_t** out);
hipError_t launch_attn_fwd_fp8(const KGeom& g, const uint8_t* q8, const float* qs, const uint8_t* k8,
                               const float* ks, const uint8_t* v8t, const float* vs, const int32_t* idx, int topk,
                               float scale, bool raster_out, uint16_t* o, float* lse, hipStream_t s);
// The fp8 stage on packed tiles: K codes in compact rows (k8c), V codes in the
// slot layout (v8s); ws as launch_attn_fwd_packed's.
hipError_t launch_attn_fwd_fp8_packed(const KGeom& g, const uint8_t* q8, const float* qs, const uint8_t* k8c,
                                      const float* ks, const uint8_t* v8s, const float* vs, const int32_t* idx,
                                      int topk, float scale, bool raster_out, uint16_t* o, float* lse, void* ws,
                                      hipStream_t s);
hipError_t launch_attn_bwd(const KGeom& g, const uint16_t* qc, const uint16_t* kc, const uint16_t* vc,
                           const uint16_t* oc, const uint16_t* doc, const float* lse, const int32_t* idx, int topk,
                           float scale, uint16_t* dq, uint16_t* dk, uint16_t* dv, void* ws, hipStream_t s);
}  // namespace vsa
