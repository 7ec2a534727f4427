"""fp64 CPU oracle for cube block-sparse video attention (forward).

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import this module.  The product path (the
HIP library and its Python binding) never calls it, and this module imports
nothing from the product package: the two share no code.

What is computed, and where it comes from
-----------------------------------------
The pages describe video sparse attention (VSA) as attention that picks the
important attention blocks dynamically, keeps roughly 10-20 % of the weights
at sparsity 0.8-0.9, stays compatible with flash-attention style kernels, and
(with the sliding-tile variant) avoids "mixed" partially masked blocks
(FastVideo sparse-distillation article, section "核心技术解析 / 2.
视频稀疏注意力VSA" and its figure caption; FastVideo attention-backend
article, figure comparing NATTEN, Tiled NATTEN and STA).  Sparse attention
paired with a linear-attention branch over the rest keeps global context at
97 % sparsity (SparkDiffusion article, paragraph 3, RoLA) at linear cost
(TurboDiffusion article, section "稀疏、蒸馏与全链路量化", SLA).

The pages give no formulas.  This oracle implements the plainest method that
fits them, with these conventions (each is a reading, not a quote):

  O1  tokens of the latent grid (T, H, W) are grouped into 4x4x4 cubes of 64
      tokens, so one 64x64 attention block is one whole query cube against
      one whole key cube (no mixed blocks).  Grid padded up to multiples of 4
      at the high end; padded tokens are zero and marked invalid.
      Cube c = ((t//4) * (Hp/4) + y//4) * (Wp/4) + x//4, local index
      l = ((t%4) * 4 + y%4) * 4 + x%4, cube-major row 64 c + l.
  O2  coarse stage: each cube is mean-pooled over its valid tokens.
  O3  block score s_ij = qbar_i . kbar_j (unscaled).
  O4  each query cube keeps the k key cubes of largest score; equal scores
      are broken towards the lower cube index; the list is stored ascending.
  O5  fine stage: softmax(scale * Q_i K^T) V over the valid keys of the
      selected cubes only (padded keys get -inf).
  O6  linear branch: phi(x) = elu(x) + 1; for each query cube, over the valid
      keys of the unselected cubes U,
      O_lin = phi(Q) (sum_U phi(K)^T V) / (phi(Q) . sum_U phi(K)),
      and 0 where U is empty.
  O7  output = O_sparse (+ O_lin), back in raster token order.
  O9  backward of the fine stage (the method is trainable: TurboDiffusion
      article, section "稀疏、蒸馏与全链路量化", SLA is a trainable sparse-linear
      attention; FastVideo sparse-distillation article, VSA is trained inside
      the distillation): for a scalar loss with output gradient dO, per query
      cube over its gathered keys, dV += P^T dO, dP = dO V^T,
      dS = P * (dP - rowsum(dO * O)), dQ = scale dS K, dK += scale dS^T Q.
      This is the chain rule through O5, written out; nothing on the pages
      fixes it further.
  O10 low-precision fine stage: SageAttention-style 8-bit attention
      (TurboDiffusion article, section "稀疏、蒸馏与全链路量化": the key
      matrix products of attention at 8 bits or lower, orthogonal to the
      sparsity).  Reading: fp8 E4M3 (OCP E4M3FN: bias 7, largest finite
      value 448) with Q and K scaled per (b, h, cube), V per (b, h, channel)
      over all tokens of the head; the attention itself is O5 on the
      dequantized values.  The quantizer is written in exact fp32 steps:
      inv = 448 / m, q = clamp(x * inv, -448, 448), code = RNE to E4M3, with
      m the block's largest |x| over valid tokens and the stored scale m / 448.
  O8  sliding-tile variant (STA, named among the attention backends of the
      FastVideo attention-backend article, item "SLIDING_TILE_ATTN" and the
      figure comparing NATTEN, Tiled NATTEN and STA): instead of the top-k
      list, each query cube attends to a fixed window of key cubes,
      (wt, wh, ww) cubes wide, centred on the query cube where possible and
      shifted inwards at the grid borders so that every query cube keeps the
      same number of key cubes (the whole axis when the window is wider).
      The pages name the pattern but give no window; this is the reading.

  O12 packed cube layouts (a data layout, not a step of the method; the
      pages only fix that blocks are whole cubes, so the order of tokens
      inside a cube is free): "compact" order puts a cube's valid tokens
      first, in raster order within the cube, then its padded slots, so a
      cube with n valid tokens fills rows 0 .. n-1 of its 64.  The "slots"
      layout cuts each compact cube into four 16-row slots and stores each
      slot transposed (channel-major).  For a full cube compact order is the
      O1 order.

Every step is written as its definition, in float64, with no blocking,
fusion or reordering beyond the definition.  Inputs are bf16 bit patterns
(numpy uint16); they are widened exactly to float64 here.
"""

from __future__ import annotations

import math
from typing import Optional, Sequence, Tuple

import numpy as np

__all__ = [
    "bf16_to_f64",
    "padded_grid",
    "cube_grid",
    "n_cubes",
    "token_row",
    "valid_rows",
    "cube_permute",
    "cube_unpermute",
    "compact_order",
    "cube_permute_compact",
    "cube_slots",
    "cube_means",
    "block_scores",
    "topk_row",
    "select_topk",
    "attention_cube",
    "sparse_attention",
    "phi",
    "linear_cube",
    "linear_branch",
    "linear_cube_states",
    "unselected_sums",
    "forward",
    "sta_window",
    "sta_index",
    "E4M3_MAX",
    "e4m3_decode",
    "e4m3_encode",
    "quant_cubes",
    "quant_channels",
    "attention_cube_bwd",
    "sparse_attention_bwd",
    "backward",
    "phi_grad",
    "linear_branch_bwd",
]


# --------------------------------------------------------------------------
# Numbers
# --------------------------------------------------------------------------

def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to float64 exactly (bf16 is the top half of fp32)."""
    u32 = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u32.view(np.float32).astype(np.float64)


# --------------------------------------------------------------------------
# O1: cube tiling and permutation
# --------------------------------------------------------------------------

def padded_grid(grid: Sequence[int]) -> Tuple[int, int, int]:
    """Each grid axis rounded up to a multiple of 4 (padding at the high end)."""
    return tuple(((int(d) + 3) // 4) * 4 for d in grid)


def cube_grid(grid: Sequence[int]) -> Tuple[int, int, int]:
    """Number of cubes along each axis."""
    tp, hp, wp = padded_grid(grid)
    return tp // 4, hp // 4, wp // 4


def n_cubes(grid: Sequence[int]) -> int:
    a, b, c = cube_grid(grid)
    return a * b * c


def token_row(t: int, y: int, x: int, grid: Sequence[int]) -> Tuple[int, int]:
    """(cube c, local l) of the token at (t, y, x), per convention O1."""
    _, cy, cx = cube_grid(grid)
    c = ((t // 4) * cy + (y // 4)) * cx + (x // 4)
    l = ((t % 4) * 4 + (y % 4)) * 4 + (x % 4)
    return c, l


def _row_of_token(grid: Sequence[int]) -> np.ndarray:
    """Cube-major row 64 c + l of every raster token (t slowest, x fastest)."""
    T, H, W = grid
    rows = np.empty(T * H * W, dtype=np.int64)
    s = 0
    for t in range(T):
        for y in range(H):
            for x in range(W):
                c, l = token_row(t, y, x, grid)
                rows[s] = 64 * c + l
                s += 1
    return rows


def valid_rows(grid: Sequence[int]) -> np.ndarray:
    """bool[Np]: True for cube-major rows that hold a real token."""
    valid = np.zeros(n_cubes(grid) * 64, dtype=bool)
    valid[_row_of_token(grid)] = True
    return valid


def cube_permute(x: np.ndarray, grid: Sequence[int]) -> np.ndarray:
    """[B, S, H, D] raster tokens -> [B, H, Np, D] cube-major rows (O1).

    Works on any dtype (bit patterns move unchanged); padded rows are zero.
    """
    B, S, Hh, D = x.shape
    rows = _row_of_token(grid)
    assert S == rows.size, "token count does not match the grid"
    out = np.zeros((B, Hh, n_cubes(grid) * 64, D), dtype=x.dtype)
    for s in range(S):
        out[:, :, rows[s], :] = x[:, s, :, :]
    return out


def cube_unpermute(xc: np.ndarray, grid: Sequence[int]) -> np.ndarray:
    """Inverse of cube_permute: [B, H, Np, D] -> [B, S, H, D], pads dropped."""
    B, Hh, Np, D = xc.shape
    rows = _row_of_token(grid)
    out = np.zeros((B, rows.size, Hh, D), dtype=xc.dtype)
    for s in range(rows.size):
        out[:, s, :, :] = xc[:, :, rows[s], :]
    return out


def compact_order(grid: Sequence[int]) -> np.ndarray:
    """int[Nc, 64]: for each cube, its local indices l (O1) in compact order
    (O12): the valid ones ascending, then the padded ones ascending."""
    T, H, W = grid
    nct, ncy, ncx = cube_grid(grid)
    order = np.empty((n_cubes(grid), 64), dtype=np.int64)
    for ct in range(nct):
        for cy in range(ncy):
            for cx in range(ncx):
                c = (ct * ncy + cy) * ncx + cx
                real, pad = [], []
                for lt in range(4):
                    for ly in range(4):
                        for lx in range(4):
                            l = (lt * 4 + ly) * 4 + lx
                            inside = 4 * ct + lt < T and 4 * cy + ly < H and 4 * cx + lx < W
                            (real if inside else pad).append(l)
                order[c] = real + pad
    return order


def cube_permute_compact(x: np.ndarray, grid: Sequence[int]) -> np.ndarray:
    """[B, S, H, D] raster tokens -> [B, H, Np, D] cube-major rows in compact
    order (O12): row 64 c + r holds local token compact_order(grid)[c, r];
    padded rows are zero."""
    xc = cube_permute(x, grid)
    order = compact_order(grid)
    out = np.zeros_like(xc)
    for c in range(order.shape[0]):
        for r in range(64):
            out[:, :, 64 * c + r, :] = xc[:, :, 64 * c + order[c, r], :]
    return out


def cube_slots(xc_compact: np.ndarray) -> np.ndarray:
    """[B, H, Np, D] compact rows -> [B, H, Nc, 4, D, 16] (O12): element
    (c, s, d, e) is channel d of compact row 16 s + e of cube c."""
    B, Hh, Np, D = xc_compact.shape
    out = np.zeros((B, Hh, Np // 64, 4, D, 16), dtype=xc_compact.dtype)
    for c in range(Np // 64):
        for s_ in range(4):
            for e in range(16):
                out[:, :, c, s_, :, e] = xc_compact[:, :, 64 * c + 16 * s_ + e, :]
    return out


# --------------------------------------------------------------------------
# O2-O4: coarse stage
# --------------------------------------------------------------------------

def cube_means(xc: np.ndarray, valid: np.ndarray) -> np.ndarray:
    """Mean of each cube over its valid rows (O2): [B, H, Np, D] -> [B, H, Nc, D] f64."""
    x = bf16_to_f64(xc) if xc.dtype == np.uint16 else np.asarray(xc, dtype=np.float64)
    B, Hh, Np, D = x.shape
    nc = Np // 64
    out = np.zeros((B, Hh, nc, D), dtype=np.float64)
    for c in range(nc):
        rows = [64 * c + l for l in range(64) if valid[64 * c + l]]
        out[:, :, c, :] = x[:, :, rows, :].sum(axis=2) / len(rows)
    return out


def block_scores(qbar: np.ndarray, kbar: np.ndarray) -> np.ndarray:
    """s_ij = qbar_i . kbar_j, unscaled (O3): [B, H, Nc, D] x2 -> [B, H, Nc, Nc]."""
    return np.matmul(qbar, np.swapaxes(kbar, -1, -2))


def topk_row(scores: np.ndarray, k: int) -> np.ndarray:
    """The k largest scores of one row, ties to the lower index, ascending (O4).

    A stable sort on the negated score keeps equal scores in index order, so
    the first k entries are the k best with the lowest-index tie winners.
    -0.0 and +0.0 compare equal, as they should.
    """
    order = np.argsort(-np.asarray(scores, dtype=np.float64), kind="stable")
    return np.sort(order[:k]).astype(np.int32)


def select_topk(qc: np.ndarray, kc: np.ndarray, valid: np.ndarray, k: int) -> np.ndarray:
    """Block index list int32 [B, H, Nc, k] (O2-O4)."""
    qbar = cube_means(qc, valid)
    kbar = cube_means(kc, valid)
    s = block_scores(qbar, kbar)
    B, Hh, nc, _ = s.shape
    idx = np.empty((B, Hh, nc, k), dtype=np.int32)
    for b in range(B):
        for h in range(Hh):
            for i in range(nc):
                idx[b, h, i] = topk_row(s[b, h, i], k)
    return idx


# --------------------------------------------------------------------------
# O5: fine stage
# --------------------------------------------------------------------------

def _as_f64(x: np.ndarray) -> np.ndarray:
    return bf16_to_f64(x) if x.dtype == np.uint16 else np.asarray(x, dtype=np.float64)


def attention_cube(q_rows: np.ndarray, k_all: np.ndarray, v_all: np.ndarray,
                   valid: np.ndarray, cubes: Sequence[int], scale: float,
                   return_probs: bool = False):
    """Softmax attention of one query cube over the selected key cubes (O5).

    q_rows: [64, D] queries of the cube; k_all, v_all: [Np, D] of one (b, h).
    Returns O [64, D], lse [64] (natural log of the softmax normaliser, in
    units of the scaled logits) and optionally P [64, n_keys].
    """
    q = _as_f64(q_rows)
    keys = np.array([64 * j + l for j in cubes for l in range(64)], dtype=np.int64)
    kk = _as_f64(k_all[keys])
    vv = _as_f64(v_all[keys])
    logits = scale * (q @ kk.T)
    logits[:, ~valid[keys]] = -np.inf
    m = logits.max(axis=1, keepdims=True)
    e = np.exp(logits - m)
    z = e.sum(axis=1, keepdims=True)
    p = e / z
    out = p @ vv
    lse = (m + np.log(z))[:, 0]
    if return_probs:
        return out, lse, p
    return out, lse


def sparse_attention(qc, kc, vc, valid, idx, scale, cubes: Optional[Sequence[Tuple[int, int, int]]] = None):
    """O_sparse [B, H, Np, D] f64 and lse [B, H, Np] (O5).

    cubes: optional list of (b, h, i) to compute; other rows stay NaN.
    """
    B, Hh, Np, D = qc.shape
    out = np.full((B, Hh, Np, D), np.nan)
    lse = np.full((B, Hh, Np), np.nan)
    todo = cubes if cubes is not None else [
        (b, h, i) for b in range(B) for h in range(Hh) for i in range(Np // 64)]
    for b, h, i in todo:
        o, s = attention_cube(qc[b, h, 64 * i:64 * i + 64], kc[b, h], vc[b, h],
                              valid, idx[b, h, i], scale)
        out[b, h, 64 * i:64 * i + 64] = o
        lse[b, h, 64 * i:64 * i + 64] = s
    return out, lse


# --------------------------------------------------------------------------
# O6: linear branch
# --------------------------------------------------------------------------

def phi(x: np.ndarray) -> np.ndarray:
    """elu(x) + 1 with alpha = 1: x + 1 for x > 0, exp(x) otherwise."""
    x = np.asarray(x, dtype=np.float64)
    return np.where(x > 0, x + 1.0, np.exp(np.minimum(x, 0.0)))


def _cube_states(k_all: np.ndarray, v_all: np.ndarray, valid: np.ndarray):
    """Per key cube j: S_j = sum_valid phi(k)^T v  [Nc, D, D], z_j = sum_valid phi(k)  [Nc, D]."""
    kk = phi(_as_f64(k_all))
    vv = _as_f64(v_all)
    nc = kk.shape[0] // 64
    D = kk.shape[1]
    S = np.zeros((nc, D, vv.shape[1]))
    z = np.zeros((nc, D))
    for j in range(nc):
        rows = [64 * j + l for l in range(64) if valid[64 * j + l]]
        S[j] = kk[rows].T @ vv[rows]
        z[j] = kk[rows].sum(axis=0)
    return S, z


def linear_cube(q_rows: np.ndarray, states, selected: Sequence[int]) -> np.ndarray:
    """O_lin of one query cube over the unselected key cubes (O6): [64, D]."""
    S, z = states
    nc = S.shape[0]
    sel = set(int(j) for j in selected)
    unsel = [j for j in range(nc) if j not in sel]
    if not unsel:
        return np.zeros((q_rows.shape[0], S.shape[2]))
    S_u = S[unsel].sum(axis=0)
    z_u = z[unsel].sum(axis=0)
    fq = phi(_as_f64(q_rows))
    return (fq @ S_u) / (fq @ z_u)[:, None]


def linear_branch(qc, kc, vc, valid, idx, cubes: Optional[Sequence[Tuple[int, int, int]]] = None):
    """O_lin [B, H, Np, D] f64 (O6); cubes as in sparse_attention."""
    B, Hh, Np, D = qc.shape
    out = np.full((B, Hh, Np, D), np.nan)
    todo = cubes if cubes is not None else [
        (b, h, i) for b in range(B) for h in range(Hh) for i in range(Np // 64)]
    states = {}
    for b, h, i in todo:
        if (b, h) not in states:
            states[(b, h)] = _cube_states(kc[b, h], vc[b, h], valid)
        out[b, h, 64 * i:64 * i + 64] = linear_cube(qc[b, h, 64 * i:64 * i + 64],
                                                    states[(b, h)], idx[b, h, i])
    return out


def linear_cube_states(kc: np.ndarray, vc: np.ndarray, valid: np.ndarray):
    """O6's per-key-cube states of every (b, h): S [B, H, Nc, D, D] with
    S[.., j, d, e] = sum over the valid tokens r of cube j of phi(k_r)[d] v_r[e],
    and z [B, H, Nc, D], the sums of phi(k_r) over the same tokens."""
    B, Hh, Np, D = kc.shape
    nc = Np // 64
    S = np.zeros((B, Hh, nc, D, vc.shape[3]))
    z = np.zeros((B, Hh, nc, D))
    for b in range(B):
        for h in range(Hh):
            S[b, h], z[b, h] = _cube_states(kc[b, h], vc[b, h], valid)
    return S, z


def unselected_sums(S: np.ndarray, z: np.ndarray, idx: np.ndarray):
    """O6's state sums over the key cubes each query cube did not select:
    S_U [B, H, Nc, D, D] and z_U [B, H, Nc, D] (zero where every cube is
    selected).  O_lin of query row q is phi(q) S_U / (phi(q) . z_U)."""
    B, Hh, nc = S.shape[:3]
    S_u = np.zeros_like(S)
    z_u = np.zeros_like(z)
    for b in range(B):
        for h in range(Hh):
            for i in range(nc):
                sel = set(int(j) for j in idx[b, h, i])
                for j in range(nc):
                    if j not in sel:
                        S_u[b, h, i] += S[b, h, j]
                        z_u[b, h, i] += z[b, h, j]
    return S_u, z_u


# --------------------------------------------------------------------------
# O7: whole layer
# --------------------------------------------------------------------------

def forward(q: np.ndarray, k: np.ndarray, v: np.ndarray, grid: Sequence[int], topk: int,
            scale: Optional[float] = None, linear: bool = False, idx: Optional[np.ndarray] = None):
    """Whole forward: [B, S, H, D] bf16 bits -> (O [B, S, H, D] f64, idx).

    idx: optional precomputed block list (to feed a given selection).
    """
    D = q.shape[-1]
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    valid = valid_rows(grid)
    qc = cube_permute(q, grid)
    kc = cube_permute(k, grid)
    vc = cube_permute(v, grid)
    if idx is None:
        idx = select_topk(qc, kc, valid, topk)
    o, _ = sparse_attention(qc, kc, vc, valid, idx, scale)
    if linear:
        o = o + linear_branch(qc, kc, vc, valid, idx)
    return cube_unpermute(o, grid), idx


# --------------------------------------------------------------------------
# O8: sliding-tile block lists
# --------------------------------------------------------------------------

def sta_window(c: int, n: int, w: int) -> range:
    """Key-cube coordinates along one axis for query coordinate c (O8).

    w consecutive coordinates starting (w - 1) // 2 below c, shifted to stay
    inside [0, n); all n coordinates when w >= n.
    """
    if w >= n:
        return range(n)
    start = min(max(c - (w - 1) // 2, 0), n - w)
    return range(start, start + w)


def sta_index(grid: Sequence[int], window: Sequence[int]) -> np.ndarray:
    """Static block list int32 [Nc, k] of the sliding-tile pattern (O8).

    Row i lists, ascending, the key cubes (tt, yy, xx) with each coordinate in
    the window of the query cube's coordinate along that axis.
    """
    ct, ch, cw = cube_grid(grid)
    wt, wh, ww = (int(v) for v in window)
    rows = []
    for t in range(ct):
        for y in range(ch):
            for x in range(cw):
                row = [(tt * ch + yy) * cw + xx
                       for tt in sta_window(t, ct, wt)
                       for yy in sta_window(y, ch, wh)
                       for xx in sta_window(x, cw, ww)]
                rows.append(sorted(row))
    return np.asarray(rows, dtype=np.int32)


# --------------------------------------------------------------------------
# O9: backward of the fine stage
# --------------------------------------------------------------------------

def attention_cube_bwd(q_rows, k_all, v_all, valid, cubes: Sequence[int], scale: float, do_rows):
    """Gradients of O5 for one query cube (O9).

    Returns dQ [64, D], and dK, dV [n_keys, D] for the gathered keys (rows
    64 j + l for j in cubes, in that order) with the key row indices.
    """
    q = _as_f64(q_rows)
    do = _as_f64(do_rows)
    keys = np.array([64 * j + l for j in cubes for l in range(64)], dtype=np.int64)
    kk = _as_f64(k_all[keys])
    vv = _as_f64(v_all[keys])
    o, _, p = attention_cube(q_rows, k_all, v_all, valid, cubes, scale, return_probs=True)
    dv = p.T @ do
    dp = do @ vv.T
    delta = (do * o).sum(axis=1, keepdims=True)
    ds = p * (dp - delta)
    dq = scale * (ds @ kk)
    dk = scale * (ds.T @ q)
    return dq, dk, dv, keys


def sparse_attention_bwd(qc, kc, vc, valid, idx, scale, doc, heads: Optional[Sequence[Tuple[int, int]]] = None):
    """dQ, dK, dV [B, H, Np, D] f64 of O5 (O9) for cube-major inputs.

    doc: output gradient [B, H, Np, D].  heads: optional list of (b, h) to
    compute (other heads stay NaN); dK and dV of a key cube collect every
    query cube that selected it.
    """
    B, Hh, Np, D = qc.shape
    dq = np.full((B, Hh, Np, D), np.nan)
    dk = np.full((B, Hh, Np, D), np.nan)
    dv = np.full((B, Hh, Np, D), np.nan)
    todo = heads if heads is not None else [(b, h) for b in range(B) for h in range(Hh)]
    for b, h in todo:
        dk[b, h] = 0.0
        dv[b, h] = 0.0
        for i in range(Np // 64):
            gq, gk, gv, keys = attention_cube_bwd(qc[b, h, 64 * i:64 * i + 64], kc[b, h], vc[b, h], valid,
                                                  idx[b, h, i], scale, doc[b, h, 64 * i:64 * i + 64])
            dq[b, h, 64 * i:64 * i + 64] = gq
            for t, j in enumerate(idx[b, h, i]):  # key rows 64 j .. 64 j + 63 are rows 64 t .. of gk, gv
                dk[b, h, 64 * j:64 * j + 64] += gk[64 * t:64 * t + 64]
                dv[b, h, 64 * j:64 * j + 64] += gv[64 * t:64 * t + 64]
    return dq, dk, dv


def backward(q, k, v, do, grid: Sequence[int], idx: np.ndarray, scale: Optional[float] = None):
    """Whole-layer gradients (O9): raster [B, S, H, D] in, raster dQ, dK, dV f64 out.

    do: gradient of the raster output; padded rows get none.
    """
    D = q.shape[-1]
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    valid = valid_rows(grid)
    qc, kc, vc = (cube_permute(x, grid) for x in (q, k, v))
    doc = cube_permute(do, grid)
    dq, dk, dv = sparse_attention_bwd(qc, kc, vc, valid, idx, scale, doc)
    return cube_unpermute(dq, grid), cube_unpermute(dk, grid), cube_unpermute(dv, grid)


# --------------------------------------------------------------------------
# O11: backward of the linear branch
# --------------------------------------------------------------------------

def phi_grad(x: np.ndarray) -> np.ndarray:
    """d phi / dx: 1 for x > 0, exp(x) otherwise."""
    x = np.asarray(x, dtype=np.float64)
    return np.where(x > 0, 1.0, np.exp(np.minimum(x, 0.0)))


def linear_branch_bwd(qc, kc, vc, valid, idx, doc, heads: Optional[Sequence[Tuple[int, int]]] = None):
    """dQ, dK, dV [B, H, Np, D] f64 of O_lin (O6) for the output gradient doc.

    The chain rule through the steps of O6, per query cube i with unselected
    set U (nothing when U is empty, where O_lin is the constant 0):
      num = phi(Q_i) S_U, den = phi(Q_i) . z_U, O = num / den;
      dnum = dO / den, dden = -(dO . O) / den;
      d phi(Q_i) = dnum S_U^T + dden z_U^T, dS_U = phi(Q_i)^T dnum, dz_U = phi(Q_i)^T dden,
    and dS_U, dz_U flow to every key cube j of U.  Per key cube j,
    S_j = sum_r phi(k_r)^T v_r and z_j = sum_r phi(k_r) over its valid rows r give
      d phi(k_r) = dS_j v_r + dz_j, dv_r = dS_j^T phi(k_r).
    Finally dQ = d phi(Q) * phi'(Q), dK = d phi(K) * phi'(K); padded rows get
    none.  heads: optional list of (b, h) to compute (others stay NaN).
    """
    B, Hh, Np, D = qc.shape
    nc = Np // 64
    dq = np.full((B, Hh, Np, D), np.nan)
    dk = np.full((B, Hh, Np, D), np.nan)
    dv = np.full((B, Hh, Np, D), np.nan)
    todo = heads if heads is not None else [(b, h) for b in range(B) for h in range(Hh)]
    vmask = valid[:, None].astype(np.float64)
    for b, h in todo:
        S, z = _cube_states(kc[b, h], vc[b, h], valid)
        dS = np.zeros_like(S)
        dz = np.zeros_like(z)
        dq[b, h] = 0.0
        for i in range(nc):
            sel = set(int(j) for j in idx[b, h, i])
            unsel = [j for j in range(nc) if j not in sel]
            if not unsel:
                continue
            rows = slice(64 * i, 64 * i + 64)
            xq = _as_f64(qc[b, h, rows])
            fq = phi(xq)
            S_u = S[unsel].sum(axis=0)
            z_u = z[unsel].sum(axis=0)
            num = fq @ S_u
            den = fq @ z_u
            o = num / den[:, None]
            g = _as_f64(doc[b, h, rows]) * vmask[rows]
            dnum = g / den[:, None]
            dden = -(g * o).sum(axis=1) / den
            dfq = dnum @ S_u.T + dden[:, None] * z_u[None, :]
            dq[b, h, rows] = dfq * phi_grad(xq) * vmask[rows]
            dS[unsel] += fq.T @ dnum
            dz[unsel] += fq.T @ dden
        xk = _as_f64(kc[b, h])
        fk = phi(xk)
        vv = _as_f64(vc[b, h])
        for j in range(nc):
            rows = slice(64 * j, 64 * j + 64)
            dfk = vv[rows] @ dS[j].T + dz[j][None, :]
            dk[b, h, rows] = dfk * phi_grad(xk[rows]) * vmask[rows]
            dv[b, h, rows] = (fk[rows] @ dS[j]) * vmask[rows]
    return dq, dk, dv


# --------------------------------------------------------------------------
# O10: 8-bit (fp8 E4M3) quantization of the fine stage's inputs
# --------------------------------------------------------------------------

E4M3_MAX = 448.0


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    """Value of OCP E4M3FN codes: sign, 4 exponent bits (bias 7), 3 mantissa
    bits; exponent 0 is subnormal (m/8 * 2^-6); S.1111.111 is NaN."""
    c = np.asarray(codes, dtype=np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 7
    val = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.power(2.0, e - 7.0))
    val = np.where((e == 15) & (m == 7), np.nan, val)
    return sign * val


# All finite non-negative E4M3 values, ascending (code 0x00 .. 0x7E).
_E4M3_POS = e4m3_decode(np.arange(0x7F))


def e4m3_encode(x: np.ndarray) -> np.ndarray:
    """Round fp32 values in [-448, 448] to the nearest E4M3 code, ties to the
    code with even mantissa (round to nearest even), by search over the value
    table.  The sign bit is kept, also when the magnitude rounds to zero."""
    x = np.asarray(x, dtype=np.float64)
    assert np.all(np.abs(x) <= E4M3_MAX), "values must be clamped to the E4M3 range"
    a = np.abs(x)
    hi = np.searchsorted(_E4M3_POS, a, side="left")  # first table value >= a
    hi = np.minimum(hi, 0x7E)
    lo = np.maximum(hi - 1, 0)
    d_lo = a - _E4M3_POS[lo]
    d_hi = _E4M3_POS[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    mag = np.where(pick_hi, hi, lo)
    mag = np.where(_E4M3_POS[hi] == a, hi, mag)
    code = np.where(np.signbit(x), mag | 0x80, mag)
    return code.astype(np.uint8)


def _quantize(x32: np.ndarray, m32: np.ndarray):
    """Codes of x32 (fp32) for block maxima m32 (fp32, broadcastable): the
    exact fp32 steps of O10."""
    with np.errstate(divide="ignore"):
        inv = np.where(m32 > 0, np.float32(E4M3_MAX) / np.where(m32 > 0, m32, np.float32(1)), np.float32(0))
    inv = inv.astype(np.float32)
    q = np.clip((x32 * inv).astype(np.float32), -np.float32(E4M3_MAX), np.float32(E4M3_MAX))
    scale = (m32 / np.float32(E4M3_MAX)).astype(np.float32)
    return e4m3_encode(q), scale


def quant_cubes(xc: np.ndarray, valid: np.ndarray):
    """Per-(b, h, cube) quantization of cube-major rows (O10).

    xc: [B, H, Np, D] bf16 bits.  Returns codes uint8 [B, H, Np, D] (padded
    rows 0) and scale fp32 [B, H, Nc] (dequantized value = decode(code) * scale).
    """
    B, Hh, Np, D = xc.shape
    x = bf16_to_f64(xc).astype(np.float32)
    x[:, :, ~valid] = 0.0
    m = np.abs(x).reshape(B, Hh, Np // 64, 64 * D).max(axis=-1).astype(np.float32)
    mrow = np.repeat(m, 64, axis=2)[..., None]
    codes, _ = _quantize(x, mrow)
    codes[:, :, ~valid] = 0
    return codes, (m / np.float32(E4M3_MAX)).astype(np.float32)


def quant_channels(xc: np.ndarray, valid: np.ndarray):
    """Per-(b, h, channel) quantization over all valid rows of a head (O10).

    Returns codes uint8 [B, H, Np, D] (padded rows 0) and scale fp32 [B, H, D].
    """
    x = bf16_to_f64(xc).astype(np.float32)
    x[:, :, ~valid] = 0.0
    m = np.abs(x).max(axis=2).astype(np.float32)  # [B, H, D]
    codes, _ = _quantize(x, m[:, :, None, :])
    codes[:, :, ~valid] = 0
    return codes, (m / np.float32(E4M3_MAX)).astype(np.float32)
