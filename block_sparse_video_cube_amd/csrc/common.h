// Host launchers of the gfx950 kernels and the geometry conversion from the C ABI.
#pragma once

#include "device.h"
#include "vsa_cube.h"

namespace vsa {
KGeom make_kgeom(const vsa_geom& g, const vsa_dims& d);
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
// Linear branch through per-cube states (linear_states.hip): the states
// [B, H, D + 1, Nc, D] bf16 of every key cube, the summed states of the
// unselected cubes [B, H, Nc, D * D + D] bf16 of every query cube (ws: the
// selection bits, linear_unsel_workspace_bytes), and the fine stage that adds
// phi(Q) S_U / (phi(Q) . z_U) in its epilogue (q and o raster or cube-major;
// kc cube-major token rows, vt cube-transposed).
size_t linear_states_bytes(const KGeom& g);
size_t linear_unsel_bytes(const KGeom& g);
size_t linear_unsel_workspace_bytes(const KGeom& g);
hipError_t launch_lin_cube_states(const KGeom& g, const uint16_t* kc, const uint16_t* vt, uint16_t* st,
                                  hipStream_t s);
hipError_t launch_lin_unselected(const KGeom& g, const uint16_t* st, const int32_t* idx, int topk, uint16_t* su,
                                 void* ws, hipStream_t s);
hipError_t launch_attn_fwd_linear(const KGeom& g, const uint16_t* q, bool raster, const uint16_t* kc,
                                  const uint16_t* vt, const int32_t* idx, int topk, float scale, const uint16_t* su,
                                  uint16_t* o, float* lse, hipStream_t s);
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
