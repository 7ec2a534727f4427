/*
 * vsa_cube.h - C ABI of the cube block-sparse video attention library (gfx950).
 *
 * The method: video sparse attention (VSA) keeps only the important attention
 * blocks, chosen dynamically, computing about 10-20 % of the attention
 * weights at sparsity 0.8-0.9 (FastVideo sparse-distillation article,
 * section "核心技术解析 / 2. 视频稀疏注意力VSA"); grouping tokens so that every
 * block is either fully kept or fully skipped avoids "mixed" blocks (same
 * article, figure comparing attention patterns; FastVideo attention-backend
 * article, figure on NATTEN / Tiled NATTEN / STA).  An optional linear
 * attention branch over the skipped blocks keeps global context at very high
 * sparsity (SparkDiffusion article, paragraph 3, RoLA; TurboDiffusion
 * article, section "稀疏、蒸馏与全链路量化", SLA).
 *
 * Conventions this library fixes (the pages give no formulas):
 *  - tokens of a latent grid T x H x W (raster order, t slowest, x fastest)
 *    are grouped into 4 x 4 x 4 cubes of 64 tokens; every grid axis is padded
 *    at its high end to a multiple of 4; padded tokens are zero and invalid;
 *  - cube c = ((t/4) * Hp/4 + y/4) * Wp/4 + x/4, local token
 *    l = ((t%4) * 4 + y%4) * 4 + x%4, cube-major row 64 c + l;
 *  - coarse stage: mean of each cube over its valid tokens, block score
 *    s_ij = qbar_i . kbar_j (unscaled), the top-k key cubes of each query
 *    cube (equal scores: lower cube index first), listed ascending;
 *  - fine stage: softmax(scale * Q_i K^T) V over the valid keys of the
 *    selected cubes (one 64 x 64 block per selected cube);
 *  - linear branch: phi(x) = elu(x) + 1, over the valid keys of the
 *    unselected cubes U: O_lin = phi(Q) (sum_U phi(K)^T V) / (phi(Q) . sum_U phi(K)),
 *    0 when U is empty; the result is O_sparse + O_lin.
 *
 * Memory and streams.  Every data pointer is a device pointer owned by the
 * caller.  The library never allocates or frees device memory, never
 * synchronises and keeps no mutable global state; calls are thread-safe.
 * Every call validates its arguments on the host first and launches nothing
 * on error; on success it enqueues its kernels on `stream` (a hipStream_t,
 * NULL = the default stream) and returns at once.  Results are valid when the
 * stream reaches that point.  bf16 values are passed as uint16_t bit
 * patterns.  All pointers must be 16-byte aligned.
 *
 * Errors are returned as vsa_status codes; NaN or Inf inputs give unspecified
 * (but memory-safe) outputs; the contents of index lists are trusted.
 */
#ifndef VSA_CUBE_H
#define VSA_CUBE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define VSA_ABI_VERSION 4

typedef enum vsa_status {
  VSA_OK = 0,
  VSA_ERR_NULL = 1,      /* a required pointer is NULL                        */
  VSA_ERR_GEOMETRY = 2,  /* non-positive or too large batch/heads/grid        */
  VSA_ERR_HEAD_DIM = 3,  /* head_dim is not 64 or 128                         */
  VSA_ERR_TOPK = 4,      /* topk outside [1, n_cubes]                         */
  VSA_ERR_ALIGN = 5,     /* a pointer is not 16-byte aligned                  */
  VSA_ERR_WORKSPACE = 6, /* workspace smaller than the *_workspace_bytes size */
  VSA_ERR_LAYOUT = 7,    /* unknown layout code                               */
  VSA_ERR_SCALE = 8,     /* softmax scale not finite and positive             */
  VSA_ERR_LAUNCH = 9,    /* a kernel launch failed (HIP error)                */
  VSA_ERR_WINDOW = 10,   /* a sliding-tile window below 1 cube on some axis   */
  VSA_ERR_SCRATCH = 11   /* problem larger than a static scratch array       */
} vsa_status;

/* Shape of one attention layer. */
typedef struct vsa_geom {
  int32_t batch;    /* B >= 1                                  */
  int32_t heads;    /* attention heads >= 1                    */
  int32_t head_dim; /* D: 64 or 128                            */
  int32_t grid_t;   /* valid latent grid (T, H, W), each >= 1  */
  int32_t grid_h;
  int32_t grid_w;
} vsa_geom;

/* Sizes derived from a vsa_geom by vsa_geom_dims. */
typedef struct vsa_dims {
  int32_t pad_t, pad_h, pad_w;       /* grid rounded up to multiples of 4 */
  int32_t cubes_t, cubes_h, cubes_w; /* cubes per axis                    */
  int32_t n_cubes;                   /* Nc                                */
  int32_t reserved;
  int64_t tokens;                    /* S = T * H * W                     */
  int64_t rows;                      /* Np = 64 * Nc                      */
} vsa_dims;

/* Layout codes of a cube-major tensor.
 * TOKEN_MAJOR: [B, heads, Np, D], element (b, h, 64 c + l, d).
 * DIM_MAJOR:   [B, heads, Nc, D, 64], element (b, h, c, d, l): each cube
 *              stored transposed.  This is the layout the value tensor must
 *              have for vsa_sparse_attn_fwd and vsa_linear_branch.
 * RASTER: not a cube-major layout; the k_layout code of
 *              vsa_sparse_attn_fwd_raster for raster-order keys.
 * TOKEN_COMPACT: [B, heads, Np, D] in compact order: row 64 c + r holds the
 *              r-th valid token of cube c (raster order within the cube) for
 *              r < n_c (its valid count), and zero for r >= n_c.  Identical to
 *              TOKEN_MAJOR for a cube without padding.  The keys of
 *              vsa_sparse_attn_fwd_packed.
 * DIM_SLOTS:   [B, heads, Nc, 4, D, 16], element (b, h, c, s, d, e) = element
 *              d of compact row 16 s + e of cube c: each cube cut into four
 *              16-row slots, each slot stored transposed.  The values of
 *              vsa_sparse_attn_fwd_packed. */
enum {
  VSA_LAYOUT_TOKEN_MAJOR = 0,
  VSA_LAYOUT_DIM_MAJOR = 1,
  VSA_LAYOUT_RASTER = 2,
  VSA_LAYOUT_TOKEN_COMPACT = 3,
  VSA_LAYOUT_DIM_SLOTS = 4
};

/* Limits: n_cubes <= VSA_MAX_CUBES, B * heads * Np * D < 2^40. */
#define VSA_MAX_CUBES 4096

/* ---------------------------------------------------------------- host only */

/* VSA_ABI_VERSION of the built library. */
int32_t vsa_abi_version(void);

/* Static English text for a status code (never NULL). */
const char* vsa_status_string(int32_t status);

/* Validates g and fills *out.  Returns VSA_ERR_NULL, VSA_ERR_GEOMETRY,
 * VSA_ERR_HEAD_DIM or VSA_OK.  Touches no device. */
int32_t vsa_geom_dims(const vsa_geom* g, vsa_dims* out);

/* Device workspace bytes needed by vsa_select_topk / vsa_linear_branch for g
 * (0 if g is invalid).  Touches no device. */
size_t vsa_select_workspace_bytes(const vsa_geom* g);
size_t vsa_linear_workspace_bytes(const vsa_geom* g);

/* -------------------------------------------------------------- entry points */

/* Cube permutation (gather): the grouping of the latent tokens into 4 x 4 x 4
 * cubes that makes every attention block a whole cube (FastVideo
 * sparse-distillation article, section "2. 视频稀疏注意力VSA" and its figure
 * of attention patterns without mixed blocks).  x: [B, S, heads, D] bf16
 * raster tokens.  xc: output, layout per `layout` (TOKEN_MAJOR, DIM_MAJOR,
 * TOKEN_COMPACT or DIM_SLOTS; else VSA_ERR_LAYOUT) with Np rows per (b, h);
 * padded rows are written as zero.  x and xc must not overlap. */
int32_t vsa_cube_permute(const vsa_geom* g, const uint16_t* x, uint16_t* xc,
                         int32_t layout, void* stream);

/* Cube permutation fused with the coarse-stage pooling (one pass over x; the
 * coarse stage summarises each cube to choose the blocks dynamically,
 * FastVideo sparse-distillation article, section "2. 视频稀疏注意力VSA"):
 * xc as vsa_cube_permute with TOKEN_MAJOR layout, and mean: output fp32
 * [B, heads, Nc, D], the mean of each cube over its valid tokens.  The fp32
 * sums are taken in one fixed order that vsa_cube_pool, vsa_quant_fp8 and the
 * pooling inside vsa_select_topk share, so all four give bit-identical means.
 * vsa_cube_permute_pool_compact: the same with xc in TOKEN_COMPACT layout. */
int32_t vsa_cube_permute_pool(const vsa_geom* g, const uint16_t* x, uint16_t* xc,
                              float* mean, void* stream);
int32_t vsa_cube_permute_pool_compact(const vsa_geom* g, const uint16_t* x, uint16_t* xc,
                                      float* mean, void* stream);

/* Inverse permutation (scatter), back to the raster token order the model
 * uses (same passage as vsa_cube_permute).  xc: [B, heads, Np, D]
 * TOKEN_MAJOR bf16; x: output [B, S, heads, D]; padded rows of xc are
 * dropped. */
int32_t vsa_cube_unpermute(const vsa_geom* g, const uint16_t* xc, uint16_t* x,
                           void* stream);

/* Coarse stage (the dynamic choice of the important blocks, keeping 1 -
 * sparsity of them: FastVideo sparse-distillation article, section
 * "2. 视频稀疏注意力VSA"): cube means of qc and kc (fp32, over valid rows),
 * block scores s_ij = qbar_i . kbar_j (fp32) and, per query cube, the topk
 * best key cubes (equal scores: lower index first; -0 and +0 equal), written
 * ascending.
 * qc, kc: [B, heads, Np, D] TOKEN_MAJOR bf16.
 * idx: output int32 [B, heads, Nc, topk].
 * ws: device workspace of at least vsa_select_workspace_bytes(g) bytes. */
int32_t vsa_select_topk(const vsa_geom* g, const uint16_t* qc, const uint16_t* kc,
                        int32_t topk, int32_t* idx, void* ws, size_t ws_bytes,
                        void* stream);

/* Cube means only: mean [B, heads, Nc, D] fp32 of the raster tokens x as
 * vsa_cube_permute_pool computes them, without writing the cube-major copy
 * (for the raster-order fine stage below, which gathers rows itself). */
int32_t vsa_cube_pool(const vsa_geom* g, const uint16_t* x, float* mean, void* stream);

/* Coarse stage from precomputed cube means (qbar, kbar: fp32 [B, heads, Nc, D],
 * e.g. from vsa_cube_permute_pool): block scores and top-k exactly as
 * vsa_select_topk.  ws: at least vsa_select_workspace_bytes(g) bytes. */
int32_t vsa_select_topk_pooled(const vsa_geom* g, const float* qbar, const float* kbar,
                               int32_t topk, int32_t* idx, void* ws, size_t ws_bytes,
                               void* stream);

/* Fine stage reading and writing raster order: as vsa_sparse_attn_fwd, but q
 * is the raster tokens [B, S, heads, D] bf16 and the output o is raster
 * [B, S, heads, D] bf16 (every token written), so the layer needs no permute
 * of Q and no unpermute (gather-on-load of the fine stage).  k_layout:
 * VSA_LAYOUT_TOKEN_MAJOR, k = kc cube-major rows as for vsa_sparse_attn_fwd,
 * or VSA_LAYOUT_RASTER, k = raster tokens whose 64-row tiles the kernel
 * gathers itself (no permute of K either).  vt stays DIM_MAJOR.  Results are
 * bit-identical to vsa_sparse_attn_fwd followed by vsa_cube_unpermute.
 * o_f32: optional fp32 output in cube-major rows [B, heads, Np, D], as the
 * oc_f32 of vsa_sparse_attn_fwd (the o_sparse input of vsa_linear_branch); o
 * may be NULL when o_f32 is given (at least one of them, else VSA_ERR_NULL).
 * lse: optional fp32 [B, heads, Np] in cube-major row order, as there.
 * Limit: S * heads * D * 2 < 2^31 bytes (32-bit buffer offsets). */
int32_t vsa_sparse_attn_fwd_raster(const vsa_geom* g, const uint16_t* q, const uint16_t* k,
                                   int32_t k_layout, const uint16_t* vt, const int32_t* idx,
                                   int32_t topk, float softmax_scale, uint16_t* o, float* o_f32,
                                   float* lse, void* stream);

/* Sliding-tile pattern (STA; FastVideo attention-backend article, item
 * "SLIDING_TILE_ATTN" and the figure comparing NATTEN, Tiled NATTEN and STA):
 * a static block list to feed vsa_sparse_attn_fwd instead of vsa_select_topk.
 * Query cube (t, y, x) attends to the key cubes whose coordinate on each axis
 * lies in a window of win_t / win_h / win_w cubes that starts (win - 1) / 2
 * below the query's coordinate, shifted inwards to stay inside the cube grid
 * (the whole axis when the window is wider than the grid).
 *
 * vsa_sta_topk returns the list length
 * k = min(win_t, cubes_t) * min(win_h, cubes_h) * min(win_w, cubes_w), or 0 for
 * an invalid geometry or a window below 1.
 *
 * vsa_sta_index writes idx int32 [B, heads, Nc, k] (the same ascending rows
 * for every (b, h)); idx is a 16-byte aligned device buffer owned by the
 * caller.  Errors: VSA_ERR_NULL, VSA_ERR_ALIGN, VSA_ERR_WINDOW, geometry
 * errors, VSA_ERR_GEOMETRY when B * heads * Nc * k >= 2^40. */
int32_t vsa_sta_topk(const vsa_geom* g, int32_t win_t, int32_t win_h, int32_t win_w);
int32_t vsa_sta_index(const vsa_geom* g, int32_t win_t, int32_t win_h, int32_t win_w,
                      int32_t* idx, void* stream);

/* Fine stage (attention over the selected blocks only, in a flash-attention
 * compatible kernel: FastVideo sparse-distillation article, section
 * "2. 视频稀疏注意力VSA"): for every (b, h, query cube i), softmax attention
 * of its 64 query rows over the valid keys of the topk key cubes
 * idx[b, h, i, :] (flash-style online softmax, fp32 accumulation, bf16
 * matrix cores).
 * qc, kc: TOKEN_MAJOR bf16; vt: DIM_MAJOR bf16; idx: int32 [B, heads, Nc, topk]
 * with entries in [0, Nc) (duplicates are computed twice).
 * softmax_scale: finite, > 0 (usually 1/sqrt(D)).
 * oc: output bf16 [B, heads, Np, D] TOKEN_MAJOR (padded query rows hold
 * finite values that unpermute drops).
 * oc_f32: optional fp32 copy of the output before rounding (NULL to skip).
 * lse: optional fp32 [B, heads, Np], max + log(sum) of the scaled logits in
 * natural-log units (NULL to skip).  The sum is taken over the bf16-rounded
 * exponentials that weight V, so lse is within ln(1 + 2^-8) of the exact
 * log-sum-exp. */
int32_t vsa_sparse_attn_fwd(const vsa_geom* g, const uint16_t* qc, const uint16_t* kc,
                            const uint16_t* vt, const int32_t* idx, int32_t topk,
                            float softmax_scale, uint16_t* oc, float* oc_f32,
                            float* lse, void* stream);

/* Packed fine stage: the result of vsa_sparse_attn_fwd (same passage) with
 * the keys of the selected cubes packed into 64-key tiles.  A selected cube
 * with n valid keys fills ceil(n / 16) slots of 16 keys; cubes of at most two
 * slots share tiles (two or four to a tile), so a cube at the edge of the
 * grid with 16 valid keys costs a quarter of a block's loads and matrix
 * work.  The per-row packing is computed on the device (one launch) into ws.
 * q: raster [B, S, heads, D] bf16 when q_layout is VSA_LAYOUT_RASTER, and o
 *    is then raster [B, S, heads, D] (padded query rows not written); or
 *    TOKEN_MAJOR qc [B, heads, Np, D] and o cube-major TOKEN_MAJOR.  Other
 *    codes: VSA_ERR_LAYOUT.
 * kc: TOKEN_COMPACT keys; vs: DIM_SLOTS values (vsa_cube_permute[_pool_compact]).
 * idx, topk, softmax_scale: as for vsa_sparse_attn_fwd; lse: optional fp32
 *    [B, heads, Np] in cube-major row order.
 * ws: at least vsa_sparse_attn_packed_workspace_bytes(g, topk) bytes
 *    (overwritten); that size is 0 when no cube of the grid holds padding, and
 *    ws may then be NULL.
 * Results agree with vsa_sparse_attn_fwd within fp32 summation order (the
 * blocks are summed in tile order); the raster and cube-major forms are
 * bit-identical to each other.  Limit: n_cubes < 2^23. */
size_t vsa_sparse_attn_packed_workspace_bytes(const vsa_geom* g, int32_t topk);
int32_t vsa_sparse_attn_fwd_packed(const vsa_geom* g, const uint16_t* q, int32_t q_layout,
                                   const uint16_t* kc, const uint16_t* vs, const int32_t* idx,
                                   int32_t topk, float softmax_scale, uint16_t* o, float* lse,
                                   void* ws, size_t ws_bytes, void* stream);

/* Low-precision fine stage (8-bit attention after SageAttention, which the
 * TurboDiffusion article's SLA builds on, section "稀疏、蒸馏与全链路量化").
 * Format: OCP fp8 E4M3 (largest finite 448).  For a block with largest |x|
 * m over its valid tokens: inv = 448 / m (0 if m = 0), code = E4M3
 * round-to-nearest-even of clamp(x * inv, -448, 448) in fp32, and
 * scale = m / 448, so that x ~ code * scale.
 *
 * vsa_quant_fp8: raster [B, S, heads, D] bf16 q, k, v ->
 *   q8, k8: codes [B, heads, Np, D] uint8 (cube-major rows, padded rows 0),
 *     qscale, kscale [B, heads, Nc] fp32, one block per (b, h, cube);
 *   v8t: codes [B, heads, Nc, D, 64] uint8 (each cube transposed, keys within
 *     a channel row in the order the fine stage consumes them: key
 *     32 t + 16 g + 8 h + e at 32 h + 16 t + 8 g + e), vscale [B, heads, D]
 *     fp32, one block per (b, h, channel) over the head;
 *   qmean, kmean: optional (may be NULL) fp32 [B, heads, Nc, D] cube means over
 *     valid tokens, bit-identical to vsa_cube_permute_pool's, for the coarse
 *     stage.
 * ws: at least vsa_quant_fp8_workspace_bytes(g) bytes of device memory,
 * overwritten (the head maxima of V).  Three launches on `stream`.
 *
 * vsa_sparse_attn_fwd_fp8: the fine stage of vsa_sparse_attn_fwd on these
 * codes with fp8 matrix products: logits scale * sq_i * sk_j * (q8 . k8),
 * fp32 online softmax, P rounded to E4M3 after scaling each row's weights so
 * that its largest lies in [2^4, 2^8], O = sv * (v8^T P) / sum(P) over the
 * rounded weights.  o: bf16 output, cube-major [B, heads, Np, D] when
 * o_layout is VSA_LAYOUT_TOKEN_MAJOR, or raster [B, S, heads, D] when it is
 * VSA_LAYOUT_RASTER (padded query rows are then not written); other values
 * give VSA_ERR_LAYOUT.  lse: optional fp32 [B, heads, Np] (cube-major rows) as
 * there.  All pointers 16-byte aligned. */
size_t vsa_quant_fp8_workspace_bytes(const vsa_geom* g);
int32_t vsa_quant_fp8(const vsa_geom* g, const uint16_t* q, const uint16_t* k, const uint16_t* v, uint8_t* q8,
                      float* qscale, uint8_t* k8, float* kscale, uint8_t* v8t, float* vscale, float* qmean,
                      float* kmean, void* ws, size_t ws_bytes, void* stream);
/* vsa_quant_fp8 for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same launches and results, with the V head maxima kept in a static
 * device array of the library instead of a caller workspace.  The array holds
 * VSA_QUANT_SCRATCH_WORDS 32-bit words (256 KB) on every device the library
 * runs on, until the process ends; its address is looked up once per device
 * (on the first call there), and no call allocates or frees memory.  The
 * launches clear the words they use (with a kernel, no memset).  Every call on
 * one device shares that array and leaves its contents behind: calls that
 * overlap on one device (several streams or threads) race, and the caller
 * must order them.  The stream's device is used (the current device for the
 * NULL stream).  Errors: as vsa_quant_fp8 (no ws arguments), and
 * VSA_ERR_SCRATCH when B * heads * D > VSA_QUANT_SCRATCH_WORDS (nothing is
 * launched); VSA_ERR_LAUNCH if the array's address cannot be obtained. */
#define VSA_QUANT_SCRATCH_WORDS 65536
int32_t vsa_quant_fp8_noalloc(const vsa_geom* g, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                              uint8_t* q8, float* qscale, uint8_t* k8, float* kscale, uint8_t* v8t,
                              float* vscale, float* qmean, float* kmean, void* stream);
int32_t vsa_sparse_attn_fwd_fp8(const vsa_geom* g, const uint8_t* q8, const float* qscale,
                                const uint8_t* k8, const float* kscale, const uint8_t* v8t,
                                const float* vscale, const int32_t* idx, int32_t topk,
                                float softmax_scale, int32_t o_layout, uint16_t* o, float* lse,
                                void* stream);

/* The low-precision fine stage on packed tiles (the same method and passage
 * as vsa_sparse_attn_fwd_fp8; tiles packed as for vsa_sparse_attn_fwd_packed:
 * a selected cube with n valid keys fills ceil(n / 16) slots of 16 keys, and
 * cubes of one or two slots share tiles; the query cubes of each head run in
 * order of their tile count).
 *
 * vsa_quant_fp8_packed: vsa_quant_fp8 with the packed stage's layouts: the
 *   same codes and scales, but k8c holds K's codes in compact cube-major rows
 *   [B, heads, Np, D] (a cube's valid tokens first, as TOKEN_COMPACT; the
 *   other rows zero) and v8s V's codes as [B, heads, Nc, 4, D, 16]: element
 *   (b, h, c, s, d, e) = the code of channel d of compact key 16 s + e of cube
 *   c (zero past its valid keys).  Arguments, workspace and errors otherwise
 *   as vsa_quant_fp8.
 * vsa_sparse_attn_fwd_fp8_packed: the fine stage of vsa_sparse_attn_fwd_fp8
 *   on those layouts (q8, scales and outputs as there).  ws: at least
 *   vsa_sparse_attn_packed_workspace_bytes(g, topk) bytes (the packing plan
 *   and the launch order; 0 and ws may be NULL for a grid without padded
 *   cubes).  Results agree with vsa_sparse_attn_fwd_fp8 within the rounding
 *   of the weights to E4M3 and the fp32 summation order (blocks are visited in
 *   tile order).  Limit: n_cubes < 2^23.  Errors as vsa_sparse_attn_fwd_fp8,
 *   and VSA_ERR_WORKSPACE. */
int32_t vsa_quant_fp8_packed(const vsa_geom* g, const uint16_t* q, const uint16_t* k,
                             const uint16_t* v, uint8_t* q8, float* qscale, uint8_t* k8c,
                             float* kscale, uint8_t* v8s, float* vscale, float* qmean,
                             float* kmean, void* ws, size_t ws_bytes, void* stream);
int32_t vsa_sparse_attn_fwd_fp8_packed(const vsa_geom* g, const uint8_t* q8, const float* qscale,
                                       const uint8_t* k8c, const float* kscale, const uint8_t* v8s,
                                       const float* vscale, const int32_t* idx, int32_t topk,
                                       float softmax_scale, int32_t o_layout, uint16_t* o,
                                       float* lse, void* ws, size_t ws_bytes, void* stream);

/* Backward of the fine stage (the gradient of vsa_sparse_attn_fwd with respect
 * to Q, K and V; VSA and SLA are trained, FastVideo sparse-distillation
 * article section "2. 视频稀疏注意力VSA", TurboDiffusion article section
 * "稀疏、蒸馏与全链路量化").  For an output gradient dO, with P the softmax
 * weights of the forward recovered from its lse:
 *   dV_j = sum_i P_ij^T dO_i,  dS_ij = P_ij * (dO_i V_j^T - rowsum(dO_i * O_i)),
 *   dQ_i = scale sum_j dS_ij K_j,  dK_j = scale sum_i dS_ij^T Q_i,
 * over the blocks (i, j) of idx.  No atomics: the result does not depend on
 * scheduling.
 * Inputs (all [B, heads, Np, D] bf16 TOKEN_MAJOR unless stated; the kernels
 * read the transposed operands out of the same tiles):
 *   qc: Q; kc: K; vc: V; oc: the forward output; doc: dO, whose padded rows
 *   must be zero (as vsa_cube_permute writes them); lse: fp32 [B, heads, Np],
 *   the forward's lse output; idx, topk: the forward's block lists (rows
 *   ascending, entries distinct).
 * Outputs (bf16 [B, heads, Np, D] TOKEN_MAJOR, fp32 accumulation): dq, dk, dv;
 * padded rows hold zero (dq: padded query rows carry no gradient).
 * ws: at least vsa_attn_bwd_workspace_bytes(g, topk) bytes.
 * Limits as vsa_select_topk (n_cubes <= VSA_MAX_CUBES). */
size_t vsa_attn_bwd_workspace_bytes(const vsa_geom* g, int32_t topk);
int32_t vsa_sparse_attn_bwd(const vsa_geom* g, const uint16_t* qc, const uint16_t* kc,
                            const uint16_t* vc, const uint16_t* oc, const uint16_t* doc,
                            const float* lse, const int32_t* idx, int32_t topk,
                            float softmax_scale, uint16_t* dq, uint16_t* dk, uint16_t* dv,
                            void* ws, size_t ws_bytes, void* stream);

/* Linear branch and combine (a linear-attention branch beside the sparse one
 * keeps the global context of the skipped blocks at linear cost:
 * SparkDiffusion article, paragraph 3, RoLA; TurboDiffusion article, section
 * "稀疏、蒸馏与全链路量化", SLA): oc = bf16(o_sparse + O_lin), O_lin over the
 * valid keys of the cubes NOT in idx[b, h, i, :] (0 when none are left).
 * qc, kc: TOKEN_MAJOR bf16; vt: DIM_MAJOR bf16; idx as for the fine stage
 * (entries distinct); o_sparse: fp32 [B, heads, Np, D] (the oc_f32 output of
 * vsa_sparse_attn_fwd); oc: output bf16 TOKEN_MAJOR.  qo_layout:
 * VSA_LAYOUT_TOKEN_MAJOR as described, or VSA_LAYOUT_RASTER: qc is then the
 * raster query tokens [B, S, heads, D] and oc the raster output
 * [B, S, heads, D] (every token written; the values are bit-identical to the
 * TOKEN_MAJOR call followed by vsa_cube_unpermute), while kc, vt, o_sparse
 * and the optional outputs stay cube-major; other codes give VSA_ERR_LAYOUT.
 * o_sparse and oc may not overlap.  o_lin, inv_den: optional outputs, both or neither (else
 * VSA_ERR_NULL): O_lin before the combine, fp32 [B, heads, Np, D], and 1/den
 * per query row, fp32 [B, heads, Np] (0 where U is empty), for
 * vsa_linear_branch_bwd to use instead of recomputing the branch.
 * ws: at least vsa_linear_workspace_bytes(g) bytes.
 * The sum over U is taken as the total minus the selected blocks while
 * topk <= n_cubes / 2, and directly over U (a complement list built in ws)
 * when more cubes are selected, so that the difference of two nearly equal
 * sums never magnifies the rounding (n_cubes <= VSA_MAX_CUBES; larger grids
 * keep the first form). */
int32_t vsa_linear_branch(const vsa_geom* g, const uint16_t* qc, int32_t qo_layout,
                          const uint16_t* kc, const uint16_t* vt, const int32_t* idx, int32_t topk,
                          const float* o_sparse, uint16_t* oc, float* o_lin, float* inv_den,
                          void* ws, size_t ws_bytes, void* stream);

/* The linear branch (the linear-attention branch beside the sparse one:
 * SparkDiffusion article, paragraph 3, RoLA; TurboDiffusion article, section
 * "稀疏、蒸馏与全链路量化", SLA) in two parts, so that the state pass (which
 * reads only K and V) can run on another stream beside the coarse and fine
 * stages:
 * vsa_linear_state computes phi(K), S_tot and z_tot of every (b, h) into ws
 * (kc TOKEN_MAJOR, vt DIM_MAJOR, as for vsa_linear_branch); ws keeps them
 * until it is overwritten.  vsa_linear_apply then runs the rest of
 * vsa_linear_branch (same arguments, without kc) on a ws that
 * vsa_linear_state filled for the same kc and vt; the pair gives results
 * bit-identical to vsa_linear_branch.  ws: at least
 * vsa_linear_workspace_bytes(g) bytes for both.  The caller orders the two
 * (vsa_linear_apply must run after vsa_linear_state completes on ws).
 * Errors as vsa_linear_branch. */
int32_t vsa_linear_state(const vsa_geom* g, const uint16_t* kc, const uint16_t* vt, void* ws,
                         size_t ws_bytes, void* stream);
int32_t vsa_linear_apply(const vsa_geom* g, const uint16_t* qc, int32_t qo_layout,
                         const uint16_t* vt, const int32_t* idx, int32_t topk,
                         const float* o_sparse, uint16_t* oc, float* o_lin, float* inv_den,
                         void* ws, size_t ws_bytes, void* stream);

/* The linear branch through summed per-cube states (the linear-attention
 * branch over the cubes the top-k left out: SparkDiffusion article, paragraph
 * 3, RoLA; TurboDiffusion article, section "稀疏、蒸馏与全链路量化", SLA).
 * For query cube i with unselected key cubes U(i):
 *   O_lin = phi(Q_i) S_U / (phi(Q_i) . z_U),  S_U = sum_{j in U(i)} S_j,
 *   S_j = phi(K_j)^T V_j over the valid keys of cube j, z_j their phi(K_j) sums.
 * Three calls, each asynchronous on `stream`, ordered by the caller:
 *
 * vsa_linear_cube_states: states [B, heads, D + 1, Nc, D] bf16 from kc
 * (TOKEN_MAJOR) and vt (DIM_MAJOR): states[b, h, e, j, d] = S_j[d, e] for
 * e < D (d the phi feature, e the value dim) and states[b, h, D, j, d] =
 * z_j[d]; fp32 sums of the bf16-rounded phi(K) and V, rounded to bf16 once.
 * vsa_linear_states_bytes(g) gives its size.
 *
 * vsa_linear_unselected: su [B, heads, Nc, D * D + D] bf16, for query cube i
 * su[.., i, e * D + d] = S_U[d, e] and su[.., i, D * D + d] = z_U[d]: the
 * states of the cubes NOT in idx[b, h, i, :] summed in fp32 (one dense 0/1
 * product per head on the matrix cores), rounded to bf16 once; all zero when
 * every cube is selected.  idx as for the fine stage (entries in 0..Nc-1; an
 * entry outside that range selects nothing).  ws: at least
 * vsa_linear_unselected_workspace_bytes(g) bytes (the selection bits);
 * vsa_linear_unselected_bytes(g) gives the size of su.
 *
 * vsa_sparse_attn_fwd_linear: the fine stage of vsa_sparse_attn_fwd with the
 * linear branch added before its one rounding: o = bf16(O_sparse + O_lin),
 * O_lin = 0 where z_U = 0.  qo_layout: VSA_LAYOUT_RASTER (q and o raster
 * [B, S, heads, D], every token written) or VSA_LAYOUT_TOKEN_MAJOR (q and o
 * cube-major rows); kc TOKEN_MAJOR, vt DIM_MAJOR, idx and softmax_scale as for
 * vsa_sparse_attn_fwd; su from vsa_linear_unselected for the same kc, vt and
 * idx; lse: optional, as for vsa_sparse_attn_fwd (the softmax branch's).
 *
 * All pointers are device memory owned by the caller (16-byte aligned); none
 * of the outputs may overlap an input.  Errors (nothing launched):
 * VSA_ERR_NULL, VSA_ERR_ALIGN, VSA_ERR_GEOMETRY / VSA_ERR_HEAD_DIM (bad g),
 * VSA_ERR_TOPK (topk outside 1..Nc), VSA_ERR_WORKSPACE (ws too small),
 * VSA_ERR_LAYOUT (qo_layout), VSA_ERR_SCALE (softmax_scale not finite and
 * positive), VSA_ERR_LAUNCH.  The sizing calls return 0 for a bad g. */
size_t vsa_linear_states_bytes(const vsa_geom* g);
size_t vsa_linear_unselected_bytes(const vsa_geom* g);
size_t vsa_linear_unselected_workspace_bytes(const vsa_geom* g);
int32_t vsa_linear_cube_states(const vsa_geom* g, const uint16_t* kc, const uint16_t* vt,
                               uint16_t* states, void* stream);
int32_t vsa_linear_unselected(const vsa_geom* g, const uint16_t* states, const int32_t* idx,
                              int32_t topk, uint16_t* su, void* ws, size_t ws_bytes, void* stream);
int32_t vsa_sparse_attn_fwd_linear(const vsa_geom* g, const uint16_t* q, int32_t qo_layout,
                                   const uint16_t* kc, const uint16_t* vt, const int32_t* idx,
                                   int32_t topk, float softmax_scale, const uint16_t* su,
                                   uint16_t* o, float* lse, void* stream);

/* Fine stage and linear branch in one pass:
 * oc = bf16(O_sparse + O_lin), the result of vsa_sparse_attn_fwd followed by
 * vsa_linear_branch, without the fp32 O_sparse round trip and without reading
 * the selected V tiles twice.  The selected-block correction of the linear
 * branch runs on the same tile pipeline as the softmax (one workgroup of 8
 * wavefronts per query cube).  qc, kc: TOKEN_MAJOR bf16; vt: DIM_MAJOR
 * bf16; idx, topk, softmax_scale as for vsa_sparse_attn_fwd; oc: output bf16
 * TOKEN_MAJOR; lse: optional fp32 [B, heads, Np], the log-sum-exp of the
 * softmax branch alone.  ws: at least vsa_linear_workspace_bytes(g) bytes
 * (overwritten: phi(K), the total state).  Three launches on `stream`.
 * The fp32 sums are those of the two-call chain, in the same order; outputs
 * can differ from it in the last bf16 bits where multiply-add contraction in
 * the final combine differs.  The linear part is the total minus the selected
 * blocks, so topk must be at most n_cubes / 2 or equal to n_cubes (else
 * VSA_ERR_TOPK; vsa_linear_branch covers the rest). */
int32_t vsa_sparse_attn_linear_fwd(const vsa_geom* g, const uint16_t* qc, const uint16_t* kc,
                                   const uint16_t* vt, const int32_t* idx, int32_t topk,
                                   float softmax_scale, uint16_t* oc, float* lse, void* ws,
                                   size_t ws_bytes, void* stream);

/* Backward of the linear branch (the branch is trained with the sparse one:
 * TurboDiffusion article, section "稀疏、蒸馏与全链路量化"; SparkDiffusion
 * article, paragraph 3): the gradients of O_lin alone, to be added to those
 * of the fine stage (vsa_sparse_attn_bwd) for the hybrid layer.  With
 * w = dO / den and c = (dO . O_lin) / den per query row (O_lin and den
 * recomputed as in vsa_linear_branch), over the unselected key rows r of a
 * query row q:
 *   dQ_q = (sum_r (w_q . v_r - c_q) phi(k_r)) * phi'(q),
 *   dK_r = (sum_q (w_q . v_r - c_q) phi(q)) * phi'(k_r),
 *   dV_r = sum_q (phi(q) . phi(k_r)) w_q,
 * phi'(x) = 1 for x > 0, e^x otherwise.  No gradient when every cube is
 * selected (O_lin is then the constant 0).
 * Inputs: qc, kc, vc, doc TOKEN_MAJOR bf16 (doc: dO, padded rows zero); vt
 * DIM_MAJOR bf16 (V); idx, topk as for vsa_linear_branch.  o_lin, inv_den:
 * optional, both or neither: the o_lin and inv_den outputs of the forward
 * vsa_linear_branch on the same inputs; w and c then come from them in one
 * pass over the rows instead of a second pass over the selected blocks, with
 * bit-identical results.  Outputs: dq, dk,
 * dv bf16 TOKEN_MAJOR, padded rows zero.  dq_add, dk_add, dv_add: optional
 * (NULL or bf16 TOKEN_MAJOR) gradients to add before the one bf16 rounding,
 * e.g. those of the fine stage for the hybrid layer; an output may alias its
 * addend.  ws: at least
 * vsa_linear_bwd_workspace_bytes(g, topk) bytes (it holds the forward's
 * linear workspace too).  n_cubes <= VSA_MAX_CUBES.  No atomics. */
size_t vsa_linear_bwd_workspace_bytes(const vsa_geom* g, int32_t topk);
int32_t vsa_linear_branch_bwd(const vsa_geom* g, const uint16_t* qc, const uint16_t* kc,
                              const uint16_t* vc, const uint16_t* vt, const int32_t* idx,
                              int32_t topk, const uint16_t* doc, const float* o_lin,
                              const float* inv_den, const uint16_t* dq_add,
                              const uint16_t* dk_add, const uint16_t* dv_add, uint16_t* dq,
                              uint16_t* dk, uint16_t* dv, void* ws, size_t ws_bytes, void* stream);

/* Matrix-core probe (measurement support, not part of the attention path):
 * the sustained rate of the bf16 matrix cores on this device, a measured
 * denominator beside the published bf16 peak, and the shader clock during it.
 * Launches `blocks` workgroups of 256 threads on `stream`; every wavefront
 * issues iters x 8 independent 32x32x16 bf16 products (32768 flops each) on
 * register operands.  sink: device fp32 [blocks * 256], overwritten with
 * checksums; clk: device uint64 [2 * blocks], per workgroup the shader-clock
 * cycles and the 100 MHz counter ticks its first wavefront spent in the loop.
 * Errors: VSA_ERR_NULL, VSA_ERR_ALIGN, VSA_ERR_GEOMETRY (blocks or iters < 1,
 * blocks > 2^20), VSA_ERR_LAUNCH. */
int32_t vsa_mfma_probe(int32_t blocks, int32_t iters, float* sink, uint64_t* clk, void* stream);

/* HBM stream probe (measurement support, not part of the attention path): the
 * rates plain streams reach on this device, a measured denominator beside the
 * published 8 TB/s for the memory-bound steps.  kind 0: copy bytes from src to
 * dst; 1: read src (dst, if not NULL, may receive one 16-byte checksum word);
 * 2: write dst (src unused, may be NULL).  Stores are nontemporal.  One launch
 * of 16384 workgroups of 256 threads on `stream`, four 16-byte words per
 * thread per round.  src, dst: device memory the caller owns, 16-byte
 * aligned; bytes: a multiple of 16, at least 16, at most 2^40.
 * Errors: VSA_ERR_LAYOUT (kind), VSA_ERR_NULL, VSA_ERR_ALIGN, VSA_ERR_GEOMETRY
 * (bytes), VSA_ERR_LAUNCH. */
int32_t vsa_hbm_probe(int32_t kind, const void* src, void* dst, size_t bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* VSA_CUBE_H */
