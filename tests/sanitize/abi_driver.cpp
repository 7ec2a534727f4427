// Host-side driver for the sanitizer build of the C ABI (AddressSanitizer +
// UndefinedBehaviorSanitizer, host code only, no device code compiled).  It
// calls the host-only functions with extreme values and every launching entry
// point with arguments that the validation must reject, so no kernel is ever
// launched and no HIP call is made.  Exit status 0 when every call returns
// the documented status; the sanitizers abort the run on any finding.
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "vsa_cube.h"

static int failures = 0;
#define EXPECT(expr, want)                                                                        \
  do {                                                                                            \
    const long long got_ = (long long)(expr);                                                     \
    if (got_ != (long long)(want)) {                                                              \
      fprintf(stderr, "line %d: %s = %lld, expected %lld\n", __LINE__, #expr, got_, (long long)(want)); \
      ++failures;                                                                                 \
    }                                                                                             \
  } while (0)

static vsa_geom geom(int32_t b, int32_t h, int32_t d, int32_t t, int32_t y, int32_t x) {
  vsa_geom g;
  g.batch = b; g.heads = h; g.head_dim = d; g.grid_t = t; g.grid_h = y; g.grid_w = x;
  return g;
}

int main() {
  // Fake device pointers: 16-byte aligned (P) or not (Q); never dereferenced.
  void* P = (void*)(uintptr_t)0x10000;
  void* Q = (void*)(uintptr_t)0x10008;
  const uint16_t* p16 = (const uint16_t*)P;
  uint16_t* w16 = (uint16_t*)P;
  const float* pf = (const float*)P;
  float* wf = (float*)P;
  const int32_t* pi = (const int32_t*)P;
  int32_t* wi = (int32_t*)P;
  uint8_t* w8 = (uint8_t*)P;
  const uint8_t* p8 = (const uint8_t*)P;

  EXPECT(vsa_abi_version(), VSA_ABI_VERSION);
  for (int32_t c = -3; c < 40; ++c) EXPECT(vsa_status_string(c) != NULL, 1);
  EXPECT(strlen(vsa_status_string(INT32_MIN)) > 0, 1);
  EXPECT(strlen(vsa_status_string(INT32_MAX)) > 0, 1);

  // Geometry: extremes of every field.
  vsa_dims d;
  const int32_t ext[] = {INT32_MIN, -1, 0, 1, 3, 4, 5, 1023, 65535, 65536, 1 << 20, INT32_MAX};
  for (int32_t a : ext)
    for (int32_t b : ext) {
      vsa_geom g = geom(1, 1, 128, a, b, 7);
      const int32_t st = vsa_geom_dims(&g, &d);
      if (a < 1 || b < 1) EXPECT(st, VSA_ERR_GEOMETRY);
      g = geom(a, b, 64, 4, 4, 4);
      const int32_t st2 = vsa_geom_dims(&g, &d);
      if (a < 1 || b < 1 || (int64_t)a * b > 65535) EXPECT(st2, VSA_ERR_GEOMETRY);
      else EXPECT(st2, VSA_OK);
      g = geom(1, 1, a, 4, 4, 4);
      EXPECT(vsa_geom_dims(&g, &d), (a == 64 || a == 128) ? VSA_OK : VSA_ERR_HEAD_DIM);
    }
  vsa_geom g = geom(1, 2, 64, 5, 6, 7);
  EXPECT(vsa_geom_dims(NULL, &d), VSA_ERR_NULL);
  EXPECT(vsa_geom_dims(&g, NULL), VSA_ERR_NULL);
  EXPECT(vsa_geom_dims(&g, &d), VSA_OK);
  EXPECT(d.n_cubes, 8);
  vsa_geom huge = geom(65535, 1, 128, INT32_MAX, INT32_MAX, INT32_MAX);
  EXPECT(vsa_geom_dims(&huge, &d), VSA_ERR_GEOMETRY);

  // Workspace sizes: zero for anything invalid, never overflowing.
  const int32_t topks[] = {INT32_MIN, -1, 0, 1, 8, 9, INT32_MAX};
  for (int32_t k : topks) {
    const bool ok = k >= 1 && k <= 8;
    EXPECT(vsa_attn_bwd_workspace_bytes(&g, k) > 0, ok);
    EXPECT(vsa_linear_bwd_workspace_bytes(&g, k) > 0, ok);
    EXPECT(vsa_sparse_attn_packed_workspace_bytes(&g, k) > 0, ok);
  }
  EXPECT(vsa_select_workspace_bytes(&huge), 0);
  EXPECT(vsa_linear_workspace_bytes(NULL), 0);
  EXPECT(vsa_quant_fp8_workspace_bytes(&huge), 0);
  vsa_geom big = geom(4, 16, 128, 255, 256, 256);  // 2^18 cubes, partial along t
  EXPECT(vsa_geom_dims(&big, &d), VSA_OK);
  EXPECT(vsa_sparse_attn_packed_workspace_bytes(&big, d.n_cubes) > (size_t)1 << 40, 1);
  vsa_geom wide = geom(8, 65, 128, 4, 4, 4);  // B * heads * D = 66560 > the static scratch
  vsa_geom full = geom(1, 2, 64, 8, 8, 8);
  EXPECT(vsa_sparse_attn_packed_workspace_bytes(&full, 3), 0);

  // Sliding-tile sizes.
  for (int32_t a : ext) {
    const int32_t k = vsa_sta_topk(&g, a, 1, INT32_MAX);
    EXPECT(k, a < 1 ? 0 : (a < 2 ? a : 2) * 1 * 2);
  }
  EXPECT(vsa_sta_index(&g, 0, 1, 1, wi, NULL), VSA_ERR_WINDOW);
  EXPECT(vsa_sta_index(&g, 1, 1, 1, (int32_t*)Q, NULL), VSA_ERR_ALIGN);
  EXPECT(vsa_sta_index(&g, 1, 1, 1, NULL, NULL), VSA_ERR_NULL);

  // Every launching entry point, rejected before any launch.
  EXPECT(vsa_cube_permute(&g, p16, w16, 5, NULL), VSA_ERR_LAYOUT);
  EXPECT(vsa_cube_permute(&g, p16, w16, -1, NULL), VSA_ERR_LAYOUT);
  EXPECT(vsa_cube_permute(&g, NULL, w16, 0, NULL), VSA_ERR_NULL);
  EXPECT(vsa_cube_permute(&g, p16, (uint16_t*)Q, 3, NULL), VSA_ERR_ALIGN);
  EXPECT(vsa_cube_permute_pool(&g, p16, w16, NULL, NULL), VSA_ERR_NULL);
  EXPECT(vsa_cube_permute_pool_compact(&g, p16, w16, (float*)Q, NULL), VSA_ERR_ALIGN);
  EXPECT(vsa_cube_pool(&huge, p16, wf, NULL), VSA_ERR_GEOMETRY);
  EXPECT(vsa_cube_unpermute(&g, p16, NULL, NULL), VSA_ERR_NULL);
  const size_t ws = vsa_select_workspace_bytes(&g);
  EXPECT(vsa_select_topk(&g, p16, p16, 9, wi, P, ws, NULL), VSA_ERR_TOPK);
  EXPECT(vsa_select_topk(&g, p16, p16, 2, wi, P, ws - 1, NULL), VSA_ERR_WORKSPACE);
  EXPECT(vsa_select_topk_pooled(&g, pf, pf, INT32_MIN, wi, P, ws, NULL), VSA_ERR_TOPK);
  EXPECT(vsa_select_topk_pooled(&big, pf, pf, 2, wi, P, (size_t)-1, NULL), VSA_ERR_GEOMETRY);
  EXPECT(vsa_sparse_attn_fwd(&g, p16, p16, p16, pi, 2, 0.f, w16, NULL, NULL, NULL), VSA_ERR_SCALE);
  EXPECT(vsa_sparse_attn_fwd(&g, p16, p16, p16, pi, 2, -1e-30f, w16, NULL, NULL, NULL), VSA_ERR_SCALE);
  EXPECT(vsa_sparse_attn_fwd(&g, p16, p16, p16, pi, INT32_MAX, 0.1f, w16, NULL, NULL, NULL), VSA_ERR_TOPK);
  EXPECT(vsa_sparse_attn_fwd(&g, p16, p16, p16, pi, 2, 0.1f, w16, (float*)Q, NULL, NULL), VSA_ERR_ALIGN);
  EXPECT(vsa_sparse_attn_fwd_raster(&g, p16, p16, 1, p16, pi, 2, 0.1f, w16, NULL, NULL, NULL), VSA_ERR_LAYOUT);
  EXPECT(vsa_sparse_attn_fwd_raster(&g, p16, p16, 0, p16, pi, 2, 0.1f, NULL, NULL, NULL, NULL), VSA_ERR_NULL);
  EXPECT(vsa_sparse_attn_fwd_packed(&g, p16, VSA_LAYOUT_RASTER, p16, p16, pi, 2, 0.1f, w16, NULL, NULL, 0, NULL),
         VSA_ERR_NULL);
  EXPECT(vsa_sparse_attn_fwd_packed(&g, p16, VSA_LAYOUT_RASTER, p16, p16, pi, 2, 0.1f, w16, NULL, P, 16, NULL),
         VSA_ERR_WORKSPACE);
  EXPECT(vsa_sparse_attn_fwd_packed(&g, p16, 4, p16, p16, pi, 2, 0.1f, w16, NULL, P, 1 << 20, NULL), VSA_ERR_LAYOUT);
  const size_t lws = vsa_linear_workspace_bytes(&g);
  EXPECT(vsa_linear_branch(&g, p16, 0, p16, p16, pi, 2, pf, w16, NULL, NULL, P, lws - 1, NULL), VSA_ERR_WORKSPACE);
  EXPECT(vsa_linear_branch(&g, p16, 3, p16, p16, pi, 2, pf, w16, NULL, NULL, P, lws, NULL), VSA_ERR_LAYOUT);
  EXPECT(vsa_linear_state(&g, p16, p16, P, lws - 1, NULL), VSA_ERR_WORKSPACE);
  EXPECT(vsa_linear_apply(&g, p16, 5, p16, pi, 2, pf, w16, NULL, NULL, P, lws, NULL), VSA_ERR_LAYOUT);
  EXPECT(vsa_linear_apply(&g, p16, 0, p16, pi, 2, pf, w16, wf, NULL, P, lws, NULL), VSA_ERR_NULL);
  EXPECT(vsa_linear_branch(&g, p16, 0, p16, p16, pi, 2, pf, w16, wf, NULL, P, lws, NULL), VSA_ERR_NULL);
  EXPECT(vsa_sparse_attn_linear_fwd(&g, p16, p16, p16, pi, 0, 0.1f, w16, NULL, P, lws, NULL), VSA_ERR_TOPK);
  const size_t bws = vsa_attn_bwd_workspace_bytes(&g, 2);
  EXPECT(vsa_sparse_attn_bwd(&g, p16, p16, p16, p16, p16, pf, pi, 2, 0.1f, w16, w16, w16, P, bws - 1, NULL),
         VSA_ERR_WORKSPACE);
  EXPECT(vsa_sparse_attn_bwd(&g, p16, p16, p16, p16, NULL, pf, pi, 2, 0.1f, w16, w16, w16, P, bws, NULL),
         VSA_ERR_NULL);
  const size_t lbws = vsa_linear_bwd_workspace_bytes(&g, 2);
  EXPECT(vsa_linear_branch_bwd(&g, p16, p16, p16, p16, pi, 2, p16, NULL, NULL, (const uint16_t*)Q, NULL, NULL, w16,
                               w16, w16, P, lbws, NULL),
         VSA_ERR_ALIGN);
  EXPECT(vsa_linear_branch_bwd(&g, p16, p16, p16, p16, pi, 2, p16, pf, NULL, NULL, NULL, NULL, w16, w16, w16, P, lbws,
                               NULL),
         VSA_ERR_NULL);
  const size_t qws = vsa_quant_fp8_workspace_bytes(&g);
  EXPECT(vsa_quant_fp8(&g, p16, p16, p16, w8, wf, w8, wf, w8, wf, NULL, NULL, P, qws - 1, NULL), VSA_ERR_WORKSPACE);
  EXPECT(vsa_quant_fp8_noalloc(&wide, p16, p16, p16, w8, wf, w8, wf, w8, wf, NULL, NULL, NULL), VSA_ERR_SCRATCH);
  EXPECT(vsa_quant_fp8_noalloc(&g, p16, NULL, p16, w8, wf, w8, wf, w8, wf, NULL, NULL, NULL), VSA_ERR_NULL);
  EXPECT(vsa_sparse_attn_fwd_fp8(&g, p8, pf, p8, pf, p8, pf, pi, 2, 0.1f, 7, w16, NULL, NULL), VSA_ERR_LAYOUT);
  EXPECT(vsa_mfma_probe(0, 1, wf, (uint64_t*)P, NULL), VSA_ERR_GEOMETRY);
  EXPECT(vsa_mfma_probe(1, INT32_MIN, wf, (uint64_t*)P, NULL), VSA_ERR_GEOMETRY);
  EXPECT(vsa_mfma_probe(INT32_MAX, 1, wf, (uint64_t*)P, NULL), VSA_ERR_GEOMETRY);
  EXPECT(vsa_hbm_probe(7, P, P, 1024, NULL), VSA_ERR_LAYOUT);
  EXPECT(vsa_hbm_probe(0, NULL, P, 1024, NULL), VSA_ERR_NULL);
  EXPECT(vsa_hbm_probe(1, P, NULL, (size_t)-16, NULL), VSA_ERR_GEOMETRY);
  EXPECT(vsa_hbm_probe(2, NULL, P, 24, NULL), VSA_ERR_GEOMETRY);

  printf("abi_driver: %d failures\n", failures);
  return failures ? 1 : 0;
}
