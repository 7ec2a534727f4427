// C ABI entry points: host-side validation, then asynchronous launches.
#include <math.h>
#include <string.h>

#include "common.h"

namespace vsa {

KGeom make_kgeom(const vsa_geom& g, const vsa_dims& d) {
  KGeom k;
  k.B = g.batch;
  k.H = g.heads;
  k.D = g.head_dim;
  k.T = g.grid_t;
  k.Hg = g.grid_h;
  k.W = g.grid_w;
  k.ct = d.cubes_t;
  k.ch = d.cubes_h;
  k.cw = d.cubes_w;
  k.nc = d.n_cubes;
  k.S = d.tokens;
  k.Np = d.rows;
  k.partial = (g.grid_t % 4 != 0) || (g.grid_h % 4 != 0) || (g.grid_w % 4 != 0);
  return k;
}

}  // namespace vsa

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int32_t launch_status(hipError_t e) { return e == hipSuccess ? VSA_OK : VSA_ERR_LAUNCH; }

// Common prologue: geometry plus the KGeom the kernels use.
int32_t prepare(const vsa_geom* g, vsa_dims* d, vsa::KGeom* k) {
  const int32_t st = vsa_geom_dims(g, d);
  if (st != VSA_OK) return st;
  *k = vsa::make_kgeom(*g, *d);
  return VSA_OK;
}

}  // namespace

extern "C" {

int32_t vsa_abi_version(void) { return VSA_ABI_VERSION; }

const char* vsa_status_string(int32_t status) {
  switch (status) {
    case VSA_OK: return "ok";
    case VSA_ERR_NULL: return "a required pointer is NULL";
    case VSA_ERR_GEOMETRY: return "invalid geometry (batch, heads or grid out of range)";
    case VSA_ERR_HEAD_DIM: return "head_dim must be 64 or 128";
    case VSA_ERR_TOPK: return "topk must lie in [1, n_cubes]";
    case VSA_ERR_ALIGN: return "pointer not 16-byte aligned";
    case VSA_ERR_WORKSPACE: return "workspace too small";
    case VSA_ERR_LAYOUT: return "unknown layout code";
    case VSA_ERR_SCALE: return "softmax scale must be finite and positive";
    case VSA_ERR_LAUNCH: return "kernel launch failed";
    case VSA_ERR_WINDOW: return "sliding-tile window must be at least 1 cube on every axis";
    case VSA_ERR_SCRATCH: return "problem larger than the library's static scratch (allocation-free entry point)";
    default: return "unknown status";
  }
}

int32_t vsa_geom_dims(const vsa_geom* g, vsa_dims* out) {
  if (!g || !out) return VSA_ERR_NULL;
  if (g->batch < 1 || g->heads < 1 || g->grid_t < 1 || g->grid_h < 1 || g->grid_w < 1)
    return VSA_ERR_GEOMETRY;
  if (g->batch > 65535 || g->heads > 65535 || (int64_t)g->batch * g->heads > 65535) return VSA_ERR_GEOMETRY;
  if (g->head_dim != 64 && g->head_dim != 128) return VSA_ERR_HEAD_DIM;
  vsa_dims d;
  memset(&d, 0, sizeof(d));
  // Cubes per axis in 64-bit, and their product checked factor by factor
  // (every factor is at least 1), so nothing overflows or narrows before the
  // n_cubes <= 2^24 limit holds.
  const int64_t lim = (int64_t)1 << 24;
  const int64_t ct = ((int64_t)g->grid_t + 3) / 4, ch = ((int64_t)g->grid_h + 3) / 4, cw = ((int64_t)g->grid_w + 3) / 4;
  if (ct > lim || ch > lim || cw > lim || ct * ch > lim || ct * ch * cw > lim) return VSA_ERR_GEOMETRY;
  const int64_t nc = ct * ch * cw;
  d.cubes_t = (int32_t)ct;
  d.cubes_h = (int32_t)ch;
  d.cubes_w = (int32_t)cw;
  d.pad_t = 4 * d.cubes_t;
  d.pad_h = 4 * d.cubes_h;
  d.pad_w = 4 * d.cubes_w;
  d.n_cubes = (int32_t)nc;
  d.tokens = (int64_t)g->grid_t * g->grid_h * g->grid_w;
  d.rows = 64 * nc;
  const int64_t elems = (int64_t)g->batch * g->heads * d.rows * g->head_dim;
  if (elems >= ((int64_t)1 << 40)) return VSA_ERR_GEOMETRY;
  *out = d;
  return VSA_OK;
}

size_t vsa_select_workspace_bytes(const vsa_geom* g) {
  vsa_dims d;
  vsa::KGeom k;
  if (prepare(g, &d, &k) != VSA_OK) return 0;
  return vsa::select_workspace_bytes(k);
}

size_t vsa_linear_workspace_bytes(const vsa_geom* g) {
  vsa_dims d;
  vsa::KGeom k;
  if (prepare(g, &d, &k) != VSA_OK) return 0;
  return vsa::linear_workspace_bytes(k);
}

int32_t vsa_cube_permute(const vsa_geom* g, const uint16_t* x, uint16_t* xc, int32_t layout, void* stream) {
  vsa_dims d;
  vsa::KGeom k;
  int32_t st = prepare(g, &d, &k);
  if (st != VSA_OK) return st;
  if (!x || !xc) return VSA_ERR_NULL;
  if (!aligned16(x) || !aligned16(xc)) return VSA_ERR_ALIGN;
  if (layout != VSA_LAYOUT_TOKEN_MAJOR && layout != VSA_LAYOUT_DIM_MAJOR && layout != VSA_LAYOUT_TOKEN_COMPACT &&
      layout != VSA_LAYOUT_DIM_SLOTS)
    return VSA_ERR_LAYOUT;
  return launch_status(vsa::launch_permute(k, x, xc, layout, static_cast<hipStream_t>(stream)));
}

int32_t vsa_cube_permute_pool(const vsa_geom* g, const uint16_t* x, uint16_t* xc, float* mean, void* stream) {
  vsa_dims d;
  vsa::KGeom k;
  int32_t st = prepare(g, &d, &k);
  if (st != VSA_OK) return st;
  if (!x || !xc || !mean) return VSA_ERR_NULL;
  if (!aligned16(x) || !aligned16(xc) || !aligned16(mean)) return VSA_ERR_ALIGN;
  return launch_status(vsa::launch_permute_pool(k, x, xc, mean, false, static_cast<hipStream_t>(stream)));
}

int32_t vsa_cube_permute_pool_compact(const vsa_geom* g, const uint16_t* x, uint16_t* xc, float* mean,
                                      void* stream) {
  vsa_dims d;
  vsa::KGeom k;
  int32_t st = prepare(g, &d, &k);
  if (st != VSA_OK) return st;
  if (!x || !xc || !mean) return VSA_ERR_NULL;
  if (!aligned16(x) || !aligned16(xc) || !aligned16(mean)) return VSA_ERR_ALIGN;
  return launch_status(vsa::launch_permute_pool(k, x, xc, mean, true, static_cast<hipStream_t>(stream)));
}

size_t vsa_sparse_attn_packed_workspace_bytes(const vsa_geom* g, int32_t topk) {
  vsa_dims d;
  vsa::KGeom k;
  if (prepare(g, &d, &k) != VSA_OK || topk < 1 || topk > d.n_cubes) return 0;
  return vsa::attn_packed_workspace_bytes(k, topk);
}

int32_t vsa_sparse_attn_fwd_packed(const vsa_geom* g, const uint16_t* q, int32_t q_layout, const uint16_t* kc,
                                   const uint16_t* vs, const int32_t* idx, int32_t topk, float softmax_scale,
                                   uint16_t* o, float* lse, void* ws, size_t ws_bytes, void* stream) {
  vsa_dims d;
  vsa::KGeom k;
  int32_t st = prepare(g, &d, &k);
  if (st != VSA_OK) return st;
  if (d.n_cubes >= (1 << 23)) return VSA_ERR_GEOMETRY;  // slot codes hold the cube index in 23 bits
  if (!q || !kc || !vs || !idx || !o) return VSA_ERR_NULL;
  if (!aligned16(q) || !aligned16(kc) || !aligned16(vs) || !aligned16(idx) || !aligned16(o) ||
      (lse && !aligned16(lse)))
    return VSA_ERR_ALIGN;
  if (q_layout != VSA_LAYOUT_TOKEN_MAJOR && q_layout != VSA_LAYOUT_RASTER) return VSA_ERR_LAYOUT;
  if (topk < 1 || topk > d.n_cubes) return VSA_ERR_TOPK;
  if (!(softmax_scale > 0.f) || !isfinite(softmax_scale)) return VSA_ERR_SCALE;
  const size_t need = vsa::attn_packed_workspace_bytes(k, topk);
  if (need) {
    if (!ws) return VSA_ERR_NULL;
    if (!aligned16(ws)) return VSA_ERR_ALIGN;
    if (ws_bytes < need) return VSA_ERR_WORKSPACE;
  }
  return launch_status(vsa::launch_attn_fwd_packed(k, q, q_layout == VSA_LAYOUT_RASTER, kc, vs, idx, topk,
                                                   softmax_scale, o, lse, ws, static_cast<hipStream_t>(stream)));
}

int32_t vsa_select_topk_pooled(const vsa_geom* g, const float* qbar, const float* kbar, int32_t topk,
                               int32_t* idx, void* ws, size_t ws_bytes, void* stream) {
  vsa_dims d;
  vsa::KGeom k;
  int32_t st = prepare(g, &d, &k);
  if (st != VSA_OK) return st;
  if (d.n_cubes > VSA_MAX_CUBES) return VSA_ERR_GEOMETRY;
  if (!qbar || !kbar || !idx || !ws) return VSA_ERR_NULL;
  if (!aligned16(qbar) || !aligned16(kbar) || !aligned16(idx) || !aligned16(ws)) return VSA_ERR_ALIGN;
  if (topk < 1 || topk > d.n_cubes) return VSA_ERR_TOPK;
  if (ws_bytes < vsa::select_pooled_workspace_bytes(k)) return VSA_ERR_WORKSPACE;
  return launch_status(vsa::launch_select_pooled(k, qbar, kbar, topk, idx, static_cast<float*>(ws),
                                                 static_cast<hipStream_t>(stream)));
}

int32_t vsa_sta_topk(const vsa_geom* g, int32_t win_t, int32_t win_h, int32_t win_w) {
  vsa_dims d;
  vsa::KGeom k;
  if (prepare(g, &d, &k) != VSA_OK) return 0;
  if (win_t < 1 || win_h < 1 || win_w < 1) return 0;
  const int64_t kk = (int64_t)(win_t < d.cubes_t ? win_t : d.cubes_t) * (win_h < d.cubes_h ? win_h : d.cubes_h) *
                     (win_w < d.cubes_w ? win_w : d.cubes_w);
  return (int32_t)kk;  // <= n_cubes <= 2^24
}

int32_t vsa_sta_index(const vsa_geom* g, int32_t win_t, int32_t win_h, int32_t win_w, int32_t* idx, void* stream) {
  vsa_dims d;
  vsa::KGeom k;
  int32_t st = prepare(g, &d, &k);
  if (st != VSA_OK) return st;
  if (!idx) return VSA_ERR_NULL;
  if (!aligned16(idx)) return VSA_ERR_ALIGN;
  if (win_t < 1 || win_h < 1 || win_w < 1) return VSA_ERR_WINDOW;
  const int64_t kk = vsa_sta_topk(g, win_t, win_h, win_w);
  if ((int64_t)g->batch * g->heads * d.n_cubes * kk >= ((int64_t)1 << 40)) return VSA_ERR_GEOMETRY;
  return launch_status(vsa::launch_sta_index(k, win_t, win_h, win_w, idx, static_cast<hipStream_t>(stream)));
}

size_t vsa_attn_bwd_workspace_bytes(const vsa_geom* g, int32_t topk) {
  vsa_dims d;
  vsa::KGeom k;
  if (prepare(g, &d, &k) != VSA_OK || topk < 1 || topk > d.n_cubes) return 0;
  return vsa::attn_bwd_workspace_bytes(k, topk);
}

int32_t vsa_sparse_attn_bwd(const vsa_geom* g, const uint16_t* qc, const uint16_t* kc, const uint16_t* vc,
                            const uint16_t* oc, const uint16_t* doc, const float* lse, const int32_t* idx,
                            int32_t topk, float softmax_scale, uint16_t* dq, uint16_t* dk, uint16_t* dv, void* ws,
                            size_t ws_bytes, void* stream) {
  vsa_dims d;
  vsa::KGeom k;
  int32_t st = prepare(g, &d, &k);
  if (st != VSA_OK) return st;
  if (d.n_cubes > VSA_MAX_CUBES) return VSA_ERR_GEOMETRY;
  const void* ptrs[] = {qc, kc, vc, oc, doc, lse, idx, dq, dk, dv, ws};
  for (const void* p : ptrs)
    if (!p) return VSA_ERR_NULL;
  for (const void* p : ptrs)
    if (!aligned16(p)) return VSA_ERR_ALIGN;
  if (topk < 1 || topk > d.n_cubes) return VSA_ERR_TOPK;
  if (!(softmax_scale > 0.f) || !isfinite(softmax_scale)) return VSA_ERR_SCALE;
  if (ws_bytes < vsa::attn_bwd_workspace_bytes(k, topk)) return VSA_ERR_WORKSPACE;
  return launch_status(vsa::launch_attn_bwd(k, qc, kc, vc, oc, doc, lse, idx, topk, softmax_scale, dq, dk, dv, ws,
                                            static_cast<hipStream_t>(stream)));
}

size_t vsa_quant_fp8_workspace_bytes(const vsa_geom* g) {
  vsa_dims d;
  vsa::KGeom k;
  if (prepare(g, &d, &k) != VSA_OK) return 0;
  return vsa::quant_workspace_bytes(k);
}

int32_t vsa_quant_fp8(const vsa_geom* g, const uint16_t* q, const uint16_t* k, const uint16_t* v, uint8_t* q8,
                      float* qscale, uint8_t* k8, float* kscale, uint8_t* v8t, float* vscale, float* qmean,
                      float* kmean, void* ws, size_t ws_bytes, void* stream) {
  vsa_dims d;
  vsa::KGeom kg;
  int32_t st = prepare(g, &d, &kg);
  if (st != VSA_OK) return st;
  const void* ptrs[] = {q, k, v, q8, qscale, k8, kscale, v8t, vscale, ws};
  for (const void* p : ptrs)
    if (!p) return VSA_ERR_NULL;
  for (const void* p : ptrs)
    if (!aligned16(p)) return VSA_ERR_ALIGN;
  if ((qmean && !aligned16(qmean)) || (kmean && !aligned16(kmean))) return VSA_ERR_ALIGN;
  if (ws_bytes < vsa::quant_workspace_bytes(kg)) return VSA_ERR_WORKSPACE;
  return launch_status(vsa::launch_quant(kg, q, k, v, q8, qscale, k8, kscale, v8t, vscale, qmean, kmean, ws,
                                         static_cast<hipStream_t>(stream)));
}

int32_t vsa_quant_fp8_packed(const vsa_geom* g, const uint16_t* q, const uint16_t* k, const uint16_t* v, uint8_t* q8,
                             float* qscale, uint8_t* k8c, float* kscale, uint8_t* v8s, float* vscale, float* qmean,
                             float* kmean, void* ws, size_t ws_bytes, void* stream) {
  vsa_dims d;
  vsa::KGeom kg;
  int32_t st = prepare(g, &d, &kg);
  if (st != VSA_OK) return st;
  const void* ptrs[] = {q, k, v, q8, qscale, k8c, kscale, v8s, vscale, ws};
  for (const void* p : ptrs)
    if (!p) return VSA_ERR_NULL;
  for (const void* p : ptrs)
    if (!aligned16(p)) return VSA_ERR_ALIGN;
  if ((qmean && !aligned16(qmean)) || (kmean && !aligned16(kmean))) return VSA_ERR_ALIGN;
  if (ws_bytes < vsa::quant_workspace_bytes(kg)) return VSA_ERR_WORKSPACE;
  return launch_status(vsa::launch_quant(kg, q, k, v, q8, qscale, k8c, kscale, v8s, vscale, qmean, kmean, ws,
                                         static_cast<hipStream_t>(stream), true));
}

int32_t vsa_quant_fp8_noalloc(const vsa_geom* g, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                              uint8_t* q8, float* qscale, uint8_t* k8, float* kscale, uint8_t* v8t, float* vscale,
                              float* qmean, float* kmean, void* stream) {
  vsa_dims d;
  vsa::KGeom kg;
  int32_t st = prepare(g, &d, &kg);
  if (st != VSA_OK) return st;
  const void* ptrs[] = {q, k, v, q8, qscale, k8, kscale, v8t, vscale};
  for (const void* p : ptrs)
    if (!p) return VSA_ERR_NULL;
  for (const void* p : ptrs)
    if (!aligned16(p)) return VSA_ERR_ALIGN;
  if ((qmean && !aligned16(qmean)) || (kmean && !aligned16(kmean))) return VSA_ERR_ALIGN;
  if ((int64_t)g->batch * g->heads * g->head_dim > VSA_QUANT_SCRATCH_WORDS) return VSA_ERR_SCRATCH;
  uint32_t* ws = nullptr;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (vsa::quant_scratch(s, &ws) != hipSuccess) return VSA_ERR_LAUNCH;
  return launch_status(vsa::launch_quant(kg, q, k, v, q8, qscale, k8, kscale, v8t, vscale, qmean, kmean, ws, s));
}

int32_t vsa_sparse_attn_fwd_fp8(const vsa_geom* g, const uint8_t* q8, const float* qscale, const uint8_t* k8,
                                const float* kscale, const uint8_t* v8t, const float* vscale, const int32_t* idx,
                                int32_t topk, float softmax_scale, int32_t o_layout, uint16_t* o, float* lse,
                                void* stream) {
  vsa_dims d;
  vsa::KGeom k;
  int32_t st = prepare(g, &d, &k);
  if (st != VSA_OK) return st;
  const void* ptrs[] = {q8, qscale, k8, kscale, v8t, vscale, idx, o};
  for (const void* p : ptrs)
    if (!p) return VSA_ERR_NULL;
  for (const void* p : ptrs)
    if (!aligned16(p)) return VSA_ERR_ALIGN;
  if (lse && !aligned16(lse)) return VSA_ERR_ALIGN;
  if (topk < 1 || topk > d.n_cubes) return VSA_ERR_TOPK;
  if (!(softmax_scale > 0.f) || !isfinite(softmax_scale)) return VSA_ERR_SCALE;
  if (o_layout != VSA_LAYOUT_TOKEN_MAJOR && o_layout != VSA_LAYOUT_RASTER) return VSA_ERR_LAYOUT;
  return launch_status(vsa::launch_attn_fwd_fp8(k, q8, qscale, k8, kscale, v8t, vscale, idx, topk, softmax_scale,
                                                o_layout == VSA_LAYOUT_RASTER, o, lse,
                                                static_cast<hipStream_t>(stream)));
}

int32_t vsa_sparse_attn_fwd_fp8_packed(const vsa_geom* g, const uint8_t* q8, const float* qscale, const uint8_t* k8c,
                                       const float* kscale, const uint8_t* v8s, const float* vscale,
                                       const int32_t* idx, int32_t topk, float softmax_scale, int32_t o_layout,
                                       uint16_t* o, float* lse, void* ws, size_t ws_bytes, void* stream) {
  vsa_dims d;
  vsa::KGeom k;
  int32_t st = prepare(g, &d, &k);
  if (st != VSA_OK) return st;
  if (d.n_cubes >= (1 << 23)) return VSA_ERR_GEOMETRY;  // slot codes hold the cube index in 23 bits
  const void* ptrs[] = {q8, qscale, k8c, kscale, v8s, vscale, idx, o};
  for (const void* p : ptrs)
    if (!p) return VSA_ERR_NULL;
  for (const void* p : ptrs)
    if (!aligned16(p)) return VSA_ERR_ALIGN;
  if (lse && !aligned16(lse)) return VSA_ERR_ALIGN;
  if (topk < 1 || topk > d.n_cubes) return VSA_ERR_TOPK;
  if (!(softmax_scale > 0.f) || !isfinite(softmax_scale)) return VSA_ERR_SCALE;
  if (o_layout != VSA_LAYOUT_TOKEN_MAJOR && o_layout != VSA_LAYOUT_RASTER) return VSA_ERR_LAYOUT;
  const size_t need = vsa::attn_packed_workspace_bytes(k, topk);
  if (need) {
    if (!ws) return VSA_ERR_NULL;
    if (!aligned16(ws)) return VSA_ERR_ALIGN;
    if (ws_bytes < need) return VSA_ERR_WORKSPACE;
  }
  return launch_status(vsa::launch_attn_fwd_fp8_packed(k, q8, qscale, k8c, kscale, v8s, vscale, idx, topk,
                                                       softmax_scale, o_layout == VSA_LAYOUT_RASTER, o, lse, ws,
                                                       static_cast<hipStream_t>(stream)));
}

int32_t vsa_cube_unpermute(const vsa_geom* g, const uint16_t* xc, uint16_t* x, void* stream) {
  vsa_dims d;
  vsa::KGeom k;
  int32_t st = prepare(g, &d, &k);
  if (st != VSA_OK) return st;
  if (!x || !xc) return VSA_ERR_NULL;
  if (!aligned16(x) || !aligned16(xc)) return VSA_ERR_ALIGN;
  return launch_status(vsa::launch_unpermute(k, xc, x, static_cast<hipStream_t>(stream)));
}

int32_t vsa_select_topk(const vsa_geom* g, const uint16_t* qc, const uint16_t* kc, int32_t topk, int32_t* idx,
                        void* ws, size_t ws_bytes, void* stream) {
  vsa_dims d;
  vsa::KGeom k;
  int32_t st = prepare(g, &d, &k);
  if (st != VSA_OK) return st;
  if (d.n_cubes > VSA_MAX_CUBES) return VSA_ERR_GEOMETRY;
  if (!qc || !kc || !idx || !ws) return VSA_ERR_NULL;
  if (!aligned16(qc) || !aligned16(kc) || !aligned16(idx) || !aligned16(ws)) return VSA_ERR_ALIGN;
  if (topk < 1 || topk > d.n_cubes) return VSA_ERR_TOPK;
  if (ws_bytes < vsa::select_workspace_bytes(k)) return VSA_ERR_WORKSPACE;
  return launch_status(vsa::launch_select(k, qc, kc, topk, idx, ws, static_cast<hipStream_t>(stream)));
}

int32_t vsa_sparse_attn_fwd_raster(const vsa_geom* g, const uint16_t* q, const uint16_t* kk, int32_t k_layout,
                                   const uint16_t* vt, const int32_t* idx, int32_t topk, float softmax_scale,
                                   uint16_t* o, float* o_f32, float* lse, void* stream) {
  vsa_dims d;
  vsa::KGeom k;
  int32_t st = prepare(g, &d, &k);
  if (st != VSA_OK) return st;
  if (!q || !kk || !vt || !idx || (!o && !o_f32)) return VSA_ERR_NULL;
  if (!aligned16(q) || !aligned16(kk) || !aligned16(vt) || !aligned16(idx) || !aligned16(o) ||
      !aligned16(o_f32) || (lse && !aligned16(lse)))
    return VSA_ERR_ALIGN;
  if (k_layout != VSA_LAYOUT_TOKEN_MAJOR && k_layout != VSA_LAYOUT_RASTER) return VSA_ERR_LAYOUT;
  if (d.tokens * (int64_t)g->heads * g->head_dim * 2 >= ((int64_t)1 << 31)) return VSA_ERR_GEOMETRY;
  if (topk < 1 || topk > d.n_cubes) return VSA_ERR_TOPK;
  if (!(softmax_scale > 0.f) || !isfinite(softmax_scale)) return VSA_ERR_SCALE;
  return launch_status(vsa::launch_attn_fwd_raster(k, q, kk, k_layout == VSA_LAYOUT_RASTER, vt, idx, topk,
                                                   softmax_scale, o, o_f32, lse, static_cast<hipStream_t>(stream)));
}

int32_t vsa_cube_pool(const vsa_geom* g, const uint16_t* x, float* mean, void* stream) {
  vsa_dims d;
  vsa::KGeom k;
  int32_t st = prepare(g, &d, &k);
  if (st != VSA_OK) return st;
  if (!x || !mean) return VSA_ERR_NULL;
  if (!aligned16(x) || !aligned16(mean)) return VSA_ERR_ALIGN;
  return launch_status(vsa::launch_permute_pool(k, x, nullptr, mean, false, static_cast<hipStream_t>(stream)));
}

int32_t vsa_sparse_attn_fwd(const vsa_geom* g, const uint16_t* qc, const uint16_t* kc, const uint16_t* vt,
                            const int32_t* idx, int32_t topk, float softmax_scale, uint16_t* oc, float* oc_f32,
                            float* lse, void* stream) {
  vsa_dims d;
  vsa::KGeom k;
  int32_t st = prepare(g, &d, &k);
  if (st != VSA_OK) return st;
  if (!qc || !kc || !vt || !idx || !oc) return VSA_ERR_NULL;
  if (!aligned16(qc) || !aligned16(kc) || !aligned16(vt) || !aligned16(idx) || !aligned16(oc) ||
      (oc_f32 && !aligned16(oc_f32)) || (lse && !aligned16(lse)))
    return VSA_ERR_ALIGN;
  if (topk < 1 || topk > d.n_cubes) return VSA_ERR_TOPK;
  if (!(softmax_scale > 0.f) || !isfinite(softmax_scale)) return VSA_ERR_SCALE;
  return launch_status(vsa::launch_attn_fwd(k, qc, kc, vt, idx, topk, softmax_scale, oc, oc_f32, lse,
                                            static_cast<hipStream_t>(stream)));
}

int32_t vsa_sparse_attn_linear_fwd(const vsa_geom* g, const uint16_t* qc, const uint16_t* kc, const uint16_t* vt,
                                   const int32_t* idx, int32_t topk, float softmax_scale, uint16_t* oc, float* lse,
                                   void* ws, size_t ws_bytes, void* stream) {
  vsa_dims d;
  vsa::KGeom k;
  int32_t st = prepare(g, &d, &k);
  if (st != VSA_OK) return st;
  if (!qc || !kc || !vt || !idx || !oc || !ws) return VSA_ERR_NULL;
  if (!aligned16(qc) || !aligned16(kc) || !aligned16(vt) || !aligned16(idx) || !aligned16(oc) || !aligned16(ws) ||
      (lse && !aligned16(lse)))
    return VSA_ERR_ALIGN;
  if (topk < 1 || topk > d.n_cubes) return VSA_ERR_TOPK;
  // The fused pass subtracts the selected blocks from the total on the
  // softmax branch's tiles; with more than half the cubes selected (and some
  // left) that difference loses precision, and vsa_linear_branch sums the
  // unselected cubes directly instead.
  if (2 * (int64_t)topk > d.n_cubes && topk < d.n_cubes) return VSA_ERR_TOPK;
  if (!(softmax_scale > 0.f) || !isfinite(softmax_scale)) return VSA_ERR_SCALE;
  if (ws_bytes < vsa::linear_workspace_bytes(k)) return VSA_ERR_WORKSPACE;
  return launch_status(vsa::launch_attn_lin_fwd(k, qc, kc, vt, idx, topk, softmax_scale, ws, oc, lse,
                                                static_cast<hipStream_t>(stream)));
}

size_t vsa_linear_bwd_workspace_bytes(const vsa_geom* g, int32_t topk) {
  vsa_dims d;
  vsa::KGeom k;
  if (prepare(g, &d, &k) != VSA_OK || topk < 1 || topk > d.n_cubes) return 0;
  return vsa::linear_bwd_workspace_bytes(k, topk);
}

int32_t vsa_linear_branch_bwd(const vsa_geom* g, const uint16_t* qc, const uint16_t* kc, const uint16_t* vc,
                              const uint16_t* vt, const int32_t* idx, int32_t topk, const uint16_t* doc,
                              const float* o_lin, const float* inv_den, const uint16_t* dq_add,
                              const uint16_t* dk_add, const uint16_t* dv_add, uint16_t* dq, uint16_t* dk, uint16_t* dv,
                              void* ws, size_t ws_bytes, void* stream) {
  vsa_dims d;
  vsa::KGeom k;
  int32_t st = prepare(g, &d, &k);
  if (st != VSA_OK) return st;
  if (d.n_cubes > VSA_MAX_CUBES) return VSA_ERR_GEOMETRY;
  const void* ptrs[] = {qc, kc, vc, vt, idx, doc, dq, dk, dv, ws};
  for (const void* p : ptrs)
    if (!p) return VSA_ERR_NULL;
  for (const void* p : ptrs)
    if (!aligned16(p)) return VSA_ERR_ALIGN;
  if ((dq_add && !aligned16(dq_add)) || (dk_add && !aligned16(dk_add)) || (dv_add && !aligned16(dv_add)))
    return VSA_ERR_ALIGN;
  if (!o_lin != !inv_den) return VSA_ERR_NULL;  // the saved forward values come as a pair
  if ((o_lin && !aligned16(o_lin)) || (inv_den && !aligned16(inv_den))) return VSA_ERR_ALIGN;
  if (topk < 1 || topk > d.n_cubes) return VSA_ERR_TOPK;
  if (ws_bytes < vsa::linear_bwd_workspace_bytes(k, topk)) return VSA_ERR_WORKSPACE;
  return launch_status(vsa::launch_linear_bwd(k, qc, kc, vc, vt, idx, topk, doc, o_lin, inv_den, dq_add, dk_add,
                                              dv_add, dq, dk, dv, ws, static_cast<hipStream_t>(stream)));
}

int32_t vsa_hbm_probe(int32_t kind, const void* src, void* dst, size_t bytes, void* stream) {
  if (kind < 0 || kind > 2) return VSA_ERR_LAYOUT;
  if ((kind != 2 && !src) || (kind != 1 && !dst)) return VSA_ERR_NULL;
  if (!aligned16(src) || !aligned16(dst)) return VSA_ERR_ALIGN;
  if (bytes < 16 || bytes % 16 != 0 || bytes > ((size_t)1 << 40)) return VSA_ERR_GEOMETRY;
  return launch_status(vsa::launch_hbm_probe(kind, src, dst, (long long)(bytes / 16), static_cast<hipStream_t>(stream)));
}

int32_t vsa_mfma_probe(int32_t blocks, int32_t iters, float* sink, uint64_t* clk, void* stream) {
  if (!sink || !clk) return VSA_ERR_NULL;
  if (!aligned16(sink) || !aligned16(clk)) return VSA_ERR_ALIGN;
  if (blocks < 1 || iters < 1 || blocks > (1 << 20)) return VSA_ERR_GEOMETRY;
  return launch_status(vsa::launch_mfma_probe(blocks, iters, sink, reinterpret_cast<unsigned long long*>(clk),
                                              static_cast<hipStream_t>(stream)));
}

int32_t vsa_linear_state(const vsa_geom* g, const uint16_t* kc, const uint16_t* vt, void* ws, size_t ws_bytes,
                         void* stream) {
  vsa_dims d;
  vsa::KGeom k;
  int32_t st = prepare(g, &d, &k);
  if (st != VSA_OK) return st;
  if (!kc || !vt || !ws) return VSA_ERR_NULL;
  if (!aligned16(kc) || !aligned16(vt) || !aligned16(ws)) return VSA_ERR_ALIGN;
  if (ws_bytes < vsa::linear_workspace_bytes(k)) return VSA_ERR_WORKSPACE;
  return launch_status(vsa::launch_lin_prep(k, kc, vt, ws, static_cast<hipStream_t>(stream)));
}

int32_t vsa_linear_apply(const vsa_geom* g, const uint16_t* qc, int32_t qo_layout, const uint16_t* vt,
                         const int32_t* idx, int32_t topk, const float* o_sparse, uint16_t* oc, float* o_lin,
                         float* inv_den, void* ws, size_t ws_bytes, void* stream) {
  vsa_dims d;
  vsa::KGeom k;
  int32_t st = prepare(g, &d, &k);
  if (st != VSA_OK) return st;
  if (!qc || !vt || !idx || !o_sparse || !oc || !ws) return VSA_ERR_NULL;
  if (!o_lin != !inv_den) return VSA_ERR_NULL;
  if (!aligned16(qc) || !aligned16(vt) || !aligned16(idx) || !aligned16(o_sparse) || !aligned16(oc) ||
      !aligned16(ws) || (o_lin && !aligned16(o_lin)) || (inv_den && !aligned16(inv_den)))
    return VSA_ERR_ALIGN;
  if (topk < 1 || topk > d.n_cubes) return VSA_ERR_TOPK;
  if (qo_layout != VSA_LAYOUT_TOKEN_MAJOR && qo_layout != VSA_LAYOUT_RASTER) return VSA_ERR_LAYOUT;
  if (ws_bytes < vsa::linear_workspace_bytes(k)) return VSA_ERR_WORKSPACE;
  return launch_status(vsa::launch_linear_apply(k, qc, vt, idx, topk, o_sparse, oc, o_lin, inv_den,
                                                qo_layout == VSA_LAYOUT_RASTER, ws, static_cast<hipStream_t>(stream)));
}

int32_t vsa_linear_branch(const vsa_geom* g, const uint16_t* qc, int32_t qo_layout, const uint16_t* kc,
                          const uint16_t* vt, const int32_t* idx, int32_t topk, const float* o_sparse, uint16_t* oc,
                          float* o_lin, float* inv_den, void* ws, size_t ws_bytes, void* stream) {
  vsa_dims d;
  vsa::KGeom k;
  int32_t st = prepare(g, &d, &k);
  if (st != VSA_OK) return st;
  if (!qc || !kc || !vt || !idx || !o_sparse || !oc || !ws) return VSA_ERR_NULL;
  if (!o_lin != !inv_den) return VSA_ERR_NULL;  // the saved values come as a pair
  if (!aligned16(qc) || !aligned16(kc) || !aligned16(vt) || !aligned16(idx) || !aligned16(o_sparse) ||
      !aligned16(oc) || !aligned16(ws))
    return VSA_ERR_ALIGN;
  if ((o_lin && !aligned16(o_lin)) || (inv_den && !aligned16(inv_den))) return VSA_ERR_ALIGN;
  if (topk < 1 || topk > d.n_cubes) return VSA_ERR_TOPK;
  if (qo_layout != VSA_LAYOUT_TOKEN_MAJOR && qo_layout != VSA_LAYOUT_RASTER) return VSA_ERR_LAYOUT;
  if (ws_bytes < vsa::linear_workspace_bytes(k)) return VSA_ERR_WORKSPACE;
  return launch_status(vsa::launch_linear(k, qc, kc, vt, idx, topk, o_sparse, oc, o_lin, inv_den,
                                          qo_layout == VSA_LAYOUT_RASTER, ws, static_cast<hipStream_t>(stream)));
}

size_t vsa_linear_states_bytes(const vsa_geom* g) {
  vsa_dims d;
  vsa::KGeom k;
  if (prepare(g, &d, &k) != VSA_OK) return 0;
  return vsa::linear_states_bytes(k);
}

size_t vsa_linear_unselected_bytes(const vsa_geom* g) {
  vsa_dims d;
  vsa::KGeom k;
  if (prepare(g, &d, &k) != VSA_OK) return 0;
  return vsa::linear_unsel_bytes(k);
}

size_t vsa_linear_unselected_workspace_bytes(const vsa_geom* g) {
  vsa_dims d;
  vsa::KGeom k;
  if (prepare(g, &d, &k) != VSA_OK) return 0;
  return vsa::linear_unsel_workspace_bytes(k);
}

int32_t vsa_linear_cube_states(const vsa_geom* g, const uint16_t* kc, const uint16_t* vt, uint16_t* states,
                               void* stream) {
  vsa_dims d;
  vsa::KGeom k;
  int32_t st = prepare(g, &d, &k);
  if (st != VSA_OK) return st;
  if (!kc || !vt || !states) return VSA_ERR_NULL;
  if (!aligned16(kc) || !aligned16(vt) || !aligned16(states)) return VSA_ERR_ALIGN;
  return launch_status(vsa::launch_lin_cube_states(k, kc, vt, states, static_cast<hipStream_t>(stream)));
}

int32_t vsa_linear_unselected(const vsa_geom* g, const uint16_t* states, const int32_t* idx, int32_t topk,
                              uint16_t* su, void* ws, size_t ws_bytes, void* stream) {
  vsa_dims d;
  vsa::KGeom k;
  int32_t st = prepare(g, &d, &k);
  if (st != VSA_OK) return st;
  if (!states || !idx || !su || !ws) return VSA_ERR_NULL;
  if (!aligned16(states) || !aligned16(idx) || !aligned16(su) || !aligned16(ws)) return VSA_ERR_ALIGN;
  if (topk < 1 || topk > d.n_cubes) return VSA_ERR_TOPK;
  if (ws_bytes < vsa::linear_unsel_workspace_bytes(k)) return VSA_ERR_WORKSPACE;
  return launch_status(vsa::launch_lin_unselected(k, states, idx, topk, su, ws, static_cast<hipStream_t>(stream)));
}

int32_t vsa_sparse_attn_fwd_linear(const vsa_geom* g, const uint16_t* q, int32_t qo_layout, const uint16_t* kc,
                                   const uint16_t* vt, const int32_t* idx, int32_t topk, float softmax_scale,
                                   const uint16_t* su, uint16_t* o, float* lse, void* stream) {
  vsa_dims d;
  vsa::KGeom k;
  int32_t st = prepare(g, &d, &k);
  if (st != VSA_OK) return st;
  if (!q || !kc || !vt || !idx || !su || !o) return VSA_ERR_NULL;
  if (!aligned16(q) || !aligned16(kc) || !aligned16(vt) || !aligned16(idx) || !aligned16(su) || !aligned16(o) ||
      (lse && !aligned16(lse)))
    return VSA_ERR_ALIGN;
  if (qo_layout != VSA_LAYOUT_TOKEN_MAJOR && qo_layout != VSA_LAYOUT_RASTER) return VSA_ERR_LAYOUT;
  if (topk < 1 || topk > d.n_cubes) return VSA_ERR_TOPK;
  if (!(softmax_scale > 0.f) || !isfinite(softmax_scale)) return VSA_ERR_SCALE;
  return launch_status(vsa::launch_attn_fwd_linear(k, q, qo_layout == VSA_LAYOUT_RASTER, kc, vt, idx, topk,
                                                   softmax_scale, su, o, lse, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
