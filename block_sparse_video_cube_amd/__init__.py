"""Cube block-sparse video attention (VSA-style) for MI355X / gfx950.

A thin binding over the C ABI in include/vsa_cube.h: every function here
only checks and marshals arguments (device pointers of torch tensors and the
current HIP stream) and calls the HIP library; all arithmetic happens in the
library's kernels.  There is no CPU fallback: if the library is missing the
calls raise.

Steps of one attention layer (q, k, v: [B, S, heads, D] bf16 on the GPU):

    qc, qbar = cube_permute_pool(q, grid)       # cube-major rows + cube means
    kc, kbar = cube_permute_pool(k, grid)
    vt = cube_permute(v, grid, layout="dim")    # cubes stored transposed
    idx = select_topk_pooled(qbar, kbar, grid, topk)  # block scores -> top-k
    oc, of, _ = sparse_attn_fwd(qc, kc, vt, idx, grid, scale, want_f32=linear)
    if linear:
        oc = linear_branch(qc, kc, vt, idx, of, grid)
    o = cube_unpermute(oc, grid)                # back to raster tokens

vsa_attention() runs them in that order.
"""

from __future__ import annotations

import math
from typing import Optional, Sequence, Tuple

import torch

from . import _lib
from ._lib import VSA_LAYOUT_DIM_MAJOR, VSA_LAYOUT_TOKEN_MAJOR, VsaDims, VsaError, VsaGeom

__all__ = [
    "VsaError",
    "make_geom",
    "geom_dims",
    "cube_permute",
    "cube_permute_pool",
    "cube_unpermute",
    "cube_pool",
    "select_topk",
    "select_topk_pooled",
    "sta_topk",
    "sta_index",
    "sparse_attn_fwd",
    "linear_branch",
    "sparse_attn_fwd_raster",
    "sparse_attn_bwd",
    "sparse_attn_linear_fwd",
    "quant_fp8",
    "quant_fp8_workspace_bytes",
    "sparse_attn_fwd_fp8",
    "vsa_attention",
    "workspace_bytes",
    "mfma_probe",
    "linear_branch_bwd",
]


def make_geom(batch: int, heads: int, head_dim: int, grid: Sequence[int]) -> VsaGeom:
    t, h, w = (int(x) for x in grid)
    return VsaGeom(int(batch), int(heads), int(head_dim), t, h, w)


def geom_dims(g: VsaGeom) -> VsaDims:
    d = VsaDims()
    _lib.check("vsa_geom_dims", _lib.load().vsa_geom_dims(g, d))
    return d


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def _need(t: torch.Tensor, name: str, dtype: torch.dtype, shape: Tuple[int, ...]) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on the GPU")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def workspace_bytes(g: VsaGeom, linear: bool = False) -> int:
    lib = _lib.load()
    return int(lib.vsa_linear_workspace_bytes(g) if linear else lib.vsa_select_workspace_bytes(g))


def cube_permute(x: torch.Tensor, grid: Sequence[int], layout: str = "token",
                 out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """[B, S, heads, D] -> [B, heads, Np, D] (layout "token") or [B, heads, Nc, D, 64] ("dim")."""
    B, S, Hh, D = x.shape
    g = make_geom(B, Hh, D, grid)
    d = geom_dims(g)
    _need(x, "x", torch.bfloat16, (B, d.tokens, Hh, D))
    code = {"token": VSA_LAYOUT_TOKEN_MAJOR, "dim": VSA_LAYOUT_DIM_MAJOR}[layout]
    shape = (B, Hh, d.rows, D) if code == VSA_LAYOUT_TOKEN_MAJOR else (B, Hh, d.n_cubes, D, 64)
    if out is None:
        out = torch.empty(shape, dtype=torch.bfloat16, device=x.device)
    _need(out, "out", torch.bfloat16, shape)
    _lib.check("vsa_cube_permute",
               _lib.load().vsa_cube_permute(g, x.data_ptr(), out.data_ptr(), code, _stream()))
    return out


def cube_permute_pool(x: torch.Tensor, grid: Sequence[int], out: Optional[torch.Tensor] = None,
                      mean_out: Optional[torch.Tensor] = None):
    """Token-major cube permutation and fp32 cube means in one pass: (xc, mean [B, heads, Nc, D])."""
    B, S, Hh, D = x.shape
    g = make_geom(B, Hh, D, grid)
    d = geom_dims(g)
    _need(x, "x", torch.bfloat16, (B, d.tokens, Hh, D))
    if out is None:
        out = torch.empty((B, Hh, d.rows, D), dtype=torch.bfloat16, device=x.device)
    if mean_out is None:
        mean_out = torch.empty((B, Hh, d.n_cubes, D), dtype=torch.float32, device=x.device)
    _need(out, "out", torch.bfloat16, (B, Hh, d.rows, D))
    _need(mean_out, "mean", torch.float32, (B, Hh, d.n_cubes, D))
    _lib.check("vsa_cube_permute_pool", _lib.load().vsa_cube_permute_pool(
        g, x.data_ptr(), out.data_ptr(), mean_out.data_ptr(), _stream()))
    return out, mean_out


def cube_pool(x: torch.Tensor, grid: Sequence[int], mean_out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """fp32 cube means [B, heads, Nc, D] of raster tokens x (no cube-major copy)."""
    B, S, Hh, D = x.shape
    g = make_geom(B, Hh, D, grid)
    d = geom_dims(g)
    _need(x, "x", torch.bfloat16, (B, d.tokens, Hh, D))
    if mean_out is None:
        mean_out = torch.empty((B, Hh, d.n_cubes, D), dtype=torch.float32, device=x.device)
    _need(mean_out, "mean", torch.float32, (B, Hh, d.n_cubes, D))
    _lib.check("vsa_cube_pool", _lib.load().vsa_cube_pool(g, x.data_ptr(), mean_out.data_ptr(), _stream()))
    return mean_out


def cube_unpermute(xc: torch.Tensor, grid: Sequence[int], out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """[B, heads, Np, D] token-major -> [B, S, heads, D]."""
    B, Hh, Np, D = xc.shape
    g = make_geom(B, Hh, D, grid)
    d = geom_dims(g)
    _need(xc, "xc", torch.bfloat16, (B, Hh, d.rows, D))
    if out is None:
        out = torch.empty((B, d.tokens, Hh, D), dtype=torch.bfloat16, device=xc.device)
    _need(out, "out", torch.bfloat16, (B, d.tokens, Hh, D))
    _lib.check("vsa_cube_unpermute",
               _lib.load().vsa_cube_unpermute(g, xc.data_ptr(), out.data_ptr(), _stream()))
    return out


def select_topk(qc: torch.Tensor, kc: torch.Tensor, grid: Sequence[int], topk: int,
                out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Block index list int32 [B, heads, Nc, topk], ascending per row."""
    B, Hh, Np, D = qc.shape
    g = make_geom(B, Hh, D, grid)
    d = geom_dims(g)
    _need(qc, "qc", torch.bfloat16, (B, Hh, d.rows, D))
    _need(kc, "kc", torch.bfloat16, (B, Hh, d.rows, D))
    if out is None:
        out = torch.empty((B, Hh, d.n_cubes, int(topk)), dtype=torch.int32, device=qc.device)
    _need(out, "idx", torch.int32, (B, Hh, d.n_cubes, int(topk)))
    nbytes = workspace_bytes(g)
    if workspace is None:
        workspace = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=qc.device)
    _lib.check("vsa_select_topk", _lib.load().vsa_select_topk(
        g, qc.data_ptr(), kc.data_ptr(), int(topk), out.data_ptr(), workspace.data_ptr(),
        workspace.numel() * workspace.element_size(), _stream()))
    return out


def select_topk_pooled(qbar: torch.Tensor, kbar: torch.Tensor, grid: Sequence[int], topk: int,
                       out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Block index list from precomputed fp32 cube means (see cube_permute_pool)."""
    B, Hh, nc, D = qbar.shape
    g = make_geom(B, Hh, D, grid)
    d = geom_dims(g)
    _need(qbar, "qbar", torch.float32, (B, Hh, d.n_cubes, D))
    _need(kbar, "kbar", torch.float32, (B, Hh, d.n_cubes, D))
    if out is None:
        out = torch.empty((B, Hh, d.n_cubes, int(topk)), dtype=torch.int32, device=qbar.device)
    _need(out, "idx", torch.int32, (B, Hh, d.n_cubes, int(topk)))
    nbytes = workspace_bytes(g)
    if workspace is None:
        workspace = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=qbar.device)
    _lib.check("vsa_select_topk_pooled", _lib.load().vsa_select_topk_pooled(
        g, qbar.data_ptr(), kbar.data_ptr(), int(topk), out.data_ptr(), workspace.data_ptr(),
        workspace.numel() * workspace.element_size(), _stream()))
    return out


def sta_topk(grid: Sequence[int], window: Sequence[int], head_dim: int = 128) -> int:
    """Length of every sliding-tile block list for this grid and window (cubes)."""
    wt, wh, ww = (int(x) for x in window)
    k = _lib.load().vsa_sta_topk(make_geom(1, 1, head_dim, grid), wt, wh, ww)
    if k < 1:
        raise VsaError("vsa_sta_topk", _lib.VSA_ERR_WINDOW, "invalid geometry or window")
    return int(k)


def sta_index(grid: Sequence[int], window: Sequence[int], batch: int, heads: int, head_dim: int = 128,
              device=None, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Static sliding-tile block list int32 [batch, heads, Nc, k] (see include/vsa_cube.h)."""
    wt, wh, ww = (int(x) for x in window)
    g = make_geom(batch, heads, head_dim, grid)
    d = geom_dims(g)
    k = sta_topk(grid, window, head_dim)
    if out is None:
        out = torch.empty((int(batch), int(heads), d.n_cubes, k), dtype=torch.int32,
                          device=device if device is not None else torch.device("cuda"))
    _need(out, "idx", torch.int32, (int(batch), int(heads), d.n_cubes, k))
    _lib.check("vsa_sta_index", _lib.load().vsa_sta_index(g, wt, wh, ww, out.data_ptr(), _stream()))
    return out


def sparse_attn_fwd(qc: torch.Tensor, kc: torch.Tensor, vt: torch.Tensor, idx: torch.Tensor,
                    grid: Sequence[int], scale: Optional[float] = None, want_f32: bool = False,
                    want_lse: bool = False, out: Optional[torch.Tensor] = None,
                    out_f32: Optional[torch.Tensor] = None):
    """Fine stage.  Returns (oc bf16, oc_f32 or None, lse or None).

    out / out_f32: optional preallocated outputs (out_f32 implies want_f32).
    """
    B, Hh, Np, D = qc.shape
    g = make_geom(B, Hh, D, grid)
    d = geom_dims(g)
    topk = idx.shape[-1]
    _need(qc, "qc", torch.bfloat16, (B, Hh, d.rows, D))
    _need(kc, "kc", torch.bfloat16, (B, Hh, d.rows, D))
    _need(vt, "vt", torch.bfloat16, (B, Hh, d.n_cubes, D, 64))
    _need(idx, "idx", torch.int32, (B, Hh, d.n_cubes, topk))
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty((B, Hh, d.rows, D), dtype=torch.bfloat16, device=qc.device)
    _need(out, "oc", torch.bfloat16, (B, Hh, d.rows, D))
    of = out_f32
    if of is None and want_f32:
        of = torch.empty((B, Hh, d.rows, D), dtype=torch.float32, device=qc.device)
    if of is not None:
        _need(of, "oc_f32", torch.float32, (B, Hh, d.rows, D))
    lse = torch.empty((B, Hh, d.rows), dtype=torch.float32, device=qc.device) if want_lse else None
    _lib.check("vsa_sparse_attn_fwd", _lib.load().vsa_sparse_attn_fwd(
        g, qc.data_ptr(), kc.data_ptr(), vt.data_ptr(), idx.data_ptr(), int(topk), float(scale),
        out.data_ptr(), of.data_ptr() if of is not None else None,
        lse.data_ptr() if lse is not None else None, _stream()))
    return out, of, lse


def sparse_attn_fwd_raster(q: torch.Tensor, k: torch.Tensor, vt: torch.Tensor, idx: torch.Tensor,
                           grid: Sequence[int], scale: Optional[float] = None, want_lse: bool = False,
                           out: Optional[torch.Tensor] = None):
    """Fine stage on raster-order q and output: returns (o [B, S, heads, D] bf16, lse or None).

    k: raster [B, S, heads, D] (tiles gathered in the kernel) or cube-major [B, heads, Np, D].
    """
    B, S, Hh, D = q.shape
    g = make_geom(B, Hh, D, grid)
    d = geom_dims(g)
    topk = int(idx.shape[-1])
    _need(q, "q", torch.bfloat16, (B, d.tokens, Hh, D))
    if tuple(k.shape) == (B, Hh, d.rows, D):
        k_layout = _lib.VSA_LAYOUT_TOKEN_MAJOR
    else:
        _need(k, "k", torch.bfloat16, (B, d.tokens, Hh, D))
        k_layout = _lib.VSA_LAYOUT_RASTER
    _need(k, "k", torch.bfloat16, tuple(k.shape))
    _need(vt, "vt", torch.bfloat16, (B, Hh, d.n_cubes, D, 64))
    _need(idx, "idx", torch.int32, (B, Hh, d.n_cubes, topk))
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty_like(q)
    _need(out, "o", torch.bfloat16, (B, d.tokens, Hh, D))
    lse = torch.empty((B, Hh, d.rows), dtype=torch.float32, device=q.device) if want_lse else None
    _lib.check("vsa_sparse_attn_fwd_raster", _lib.load().vsa_sparse_attn_fwd_raster(
        g, q.data_ptr(), k.data_ptr(), k_layout, vt.data_ptr(), idx.data_ptr(), topk, float(scale),
        out.data_ptr(), lse.data_ptr() if lse is not None else None, _stream()))
    return out, lse


def quant_fp8_workspace_bytes(g: VsaGeom) -> int:
    return int(_lib.load().vsa_quant_fp8_workspace_bytes(g))


def quant_fp8(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, grid: Sequence[int], want_means: bool = False,
              out=None, workspace: Optional[torch.Tensor] = None):
    """E4M3 codes of raster Q, K (per (b, h, cube)) and V (per (b, h, channel)).

    Returns (q8, qscale, k8, kscale, v8t, vscale, qmean, kmean): codes uint8
    [B, heads, Np, D] and [B, heads, Nc, D, 64], scales f32 [B, heads, Nc] and
    [B, heads, D], cube means f32 [B, heads, Nc, D] or None.  `out`: optional
    tuple of the same eight tensors to write into (means may be None).
    """
    B, S, Hh, D = q.shape
    g = make_geom(B, Hh, D, grid)
    d = geom_dims(g)
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, n, torch.bfloat16, (B, d.tokens, Hh, D))
    dev = q.device
    if out is None:
        u8 = dict(dtype=torch.uint8, device=dev)
        f32 = dict(dtype=torch.float32, device=dev)
        out = (torch.empty((B, Hh, d.rows, D), **u8), torch.empty((B, Hh, d.n_cubes), **f32),
               torch.empty((B, Hh, d.rows, D), **u8), torch.empty((B, Hh, d.n_cubes), **f32),
               torch.empty((B, Hh, d.n_cubes, D, 64), **u8), torch.empty((B, Hh, D), **f32),
               torch.empty((B, Hh, d.n_cubes, D), **f32) if want_means else None,
               torch.empty((B, Hh, d.n_cubes, D), **f32) if want_means else None)
    q8, qs, k8, ks, v8t, vs, qm, km = out
    _need(q8, "q8", torch.uint8, (B, Hh, d.rows, D))
    _need(k8, "k8", torch.uint8, (B, Hh, d.rows, D))
    _need(v8t, "v8t", torch.uint8, (B, Hh, d.n_cubes, D, 64))
    _need(qs, "qscale", torch.float32, (B, Hh, d.n_cubes))
    _need(ks, "kscale", torch.float32, (B, Hh, d.n_cubes))
    _need(vs, "vscale", torch.float32, (B, Hh, D))
    for t, n in ((qm, "qmean"), (km, "kmean")):
        if t is not None:
            _need(t, n, torch.float32, (B, Hh, d.n_cubes, D))
    lib = _lib.load()
    nbytes = lib.vsa_quant_fp8_workspace_bytes(g)
    if workspace is None:
        workspace = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=dev)
    _lib.check("vsa_quant_fp8", lib.vsa_quant_fp8(
        g, q.data_ptr(), k.data_ptr(), v.data_ptr(), q8.data_ptr(), qs.data_ptr(), k8.data_ptr(), ks.data_ptr(),
        v8t.data_ptr(), vs.data_ptr(), qm.data_ptr() if qm is not None else None,
        km.data_ptr() if km is not None else None, workspace.data_ptr(),
        workspace.numel() * workspace.element_size(), _stream()))
    return q8, qs, k8, ks, v8t, vs, qm, km


def sparse_attn_fwd_fp8(q8: torch.Tensor, qscale: torch.Tensor, k8: torch.Tensor, kscale: torch.Tensor,
                        v8t: torch.Tensor, vscale: torch.Tensor, idx: torch.Tensor, grid: Sequence[int],
                        scale: Optional[float] = None, want_lse: bool = False, out: Optional[torch.Tensor] = None,
                        raster: bool = False):
    """fp8 fine stage.  Returns (o bf16, lse or None): o is cube-major [B, heads, Np, D], or raster
    [B, S, heads, D] with raster=True (padded query rows not written)."""
    B, Hh, Np, D = q8.shape
    g = make_geom(B, Hh, D, grid)
    d = geom_dims(g)
    topk = int(idx.shape[-1])
    _need(q8, "q8", torch.uint8, (B, Hh, d.rows, D))
    _need(k8, "k8", torch.uint8, (B, Hh, d.rows, D))
    _need(v8t, "v8t", torch.uint8, (B, Hh, d.n_cubes, D, 64))
    _need(qscale, "qscale", torch.float32, (B, Hh, d.n_cubes))
    _need(kscale, "kscale", torch.float32, (B, Hh, d.n_cubes))
    _need(vscale, "vscale", torch.float32, (B, Hh, D))
    _need(idx, "idx", torch.int32, (B, Hh, d.n_cubes, topk))
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    oshape = (B, d.tokens, Hh, D) if raster else (B, Hh, d.rows, D)
    if out is None:
        out = torch.empty(oshape, dtype=torch.bfloat16, device=q8.device)
    _need(out, "o", torch.bfloat16, oshape)
    lse = torch.empty((B, Hh, d.rows), dtype=torch.float32, device=q8.device) if want_lse else None
    layout = _lib.VSA_LAYOUT_RASTER if raster else _lib.VSA_LAYOUT_TOKEN_MAJOR
    _lib.check("vsa_sparse_attn_fwd_fp8", _lib.load().vsa_sparse_attn_fwd_fp8(
        g, q8.data_ptr(), qscale.data_ptr(), k8.data_ptr(), kscale.data_ptr(), v8t.data_ptr(), vscale.data_ptr(),
        idx.data_ptr(), topk, float(scale), layout, out.data_ptr(), lse.data_ptr() if lse is not None else None,
        _stream()))
    return out, lse


def sparse_attn_bwd(qc: torch.Tensor, kc: torch.Tensor, vc: torch.Tensor, oc: torch.Tensor, doc: torch.Tensor,
                    lse: torch.Tensor, idx: torch.Tensor, grid: Sequence[int], scale: Optional[float] = None,
                    workspace: Optional[torch.Tensor] = None):
    """Backward of the fine stage.  Returns (dq, dk, dv), bf16 [B, heads, Np, D] token-major.

    qc, kc, vc, doc: Q, K, V and dO token-major (cube_permute); oc, lse: outputs of
    sparse_attn_fwd (want_lse=True); idx: its block lists.
    """
    B, Hh, Np, D = qc.shape
    g = make_geom(B, Hh, D, grid)
    d = geom_dims(g)
    topk = int(idx.shape[-1])
    for t, name in ((qc, "qc"), (kc, "kc"), (vc, "vc"), (oc, "oc"), (doc, "doc")):
        _need(t, name, torch.bfloat16, (B, Hh, d.rows, D))
    _need(lse, "lse", torch.float32, (B, Hh, d.rows))
    _need(idx, "idx", torch.int32, (B, Hh, d.n_cubes, topk))
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    lib = _lib.load()
    nbytes = lib.vsa_attn_bwd_workspace_bytes(g, topk)
    if workspace is None:
        workspace = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=qc.device)
    dq, dk, dv = (torch.empty_like(qc) for _ in range(3))
    _lib.check("vsa_sparse_attn_bwd", lib.vsa_sparse_attn_bwd(
        g, qc.data_ptr(), kc.data_ptr(), vc.data_ptr(), oc.data_ptr(), doc.data_ptr(), lse.data_ptr(),
        idx.data_ptr(), topk, float(scale), dq.data_ptr(),
        dk.data_ptr(), dv.data_ptr(), workspace.data_ptr(), workspace.numel() * workspace.element_size(),
        _stream()))
    return dq, dk, dv


def linear_branch(qc: torch.Tensor, kc: torch.Tensor, vt: torch.Tensor, idx: torch.Tensor,
                  o_sparse: torch.Tensor, grid: Sequence[int], out: Optional[torch.Tensor] = None,
                  workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """bf16(o_sparse + O_lin), token-major."""
    B, Hh, Np, D = qc.shape
    g = make_geom(B, Hh, D, grid)
    d = geom_dims(g)
    topk = idx.shape[-1]
    _need(qc, "qc", torch.bfloat16, (B, Hh, d.rows, D))
    _need(kc, "kc", torch.bfloat16, (B, Hh, d.rows, D))
    _need(vt, "vt", torch.bfloat16, (B, Hh, d.n_cubes, D, 64))
    _need(idx, "idx", torch.int32, (B, Hh, d.n_cubes, topk))
    _need(o_sparse, "o_sparse", torch.float32, (B, Hh, d.rows, D))
    if out is None:
        out = torch.empty((B, Hh, d.rows, D), dtype=torch.bfloat16, device=qc.device)
    _need(out, "oc", torch.bfloat16, (B, Hh, d.rows, D))
    nbytes = workspace_bytes(g, linear=True)
    if workspace is None:
        workspace = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=qc.device)
    _lib.check("vsa_linear_branch", _lib.load().vsa_linear_branch(
        g, qc.data_ptr(), kc.data_ptr(), vt.data_ptr(), idx.data_ptr(), int(topk), o_sparse.data_ptr(),
        out.data_ptr(), workspace.data_ptr(), workspace.numel() * workspace.element_size(), _stream()))
    return out


def linear_branch_bwd(qc: torch.Tensor, kc: torch.Tensor, vc: torch.Tensor, vt: torch.Tensor, idx: torch.Tensor,
                      doc: torch.Tensor, grid: Sequence[int], workspace: Optional[torch.Tensor] = None,
                      add: Optional[Tuple[torch.Tensor, torch.Tensor, torch.Tensor]] = None, out=None):
    """Gradients of the linear branch.  Returns (dq, dk, dv), bf16 [B, heads, Np, D] token-major.

    qc, kc, vc, doc: Q, K, V and dO token-major; vt: V DIM_MAJOR; idx: the block lists.
    add: optional (dq, dk, dv) added before the one bf16 rounding (the fine stage's, for the
    hybrid layer); out: optional output tensors (may be the addends themselves).
    """
    B, Hh, Np, D = qc.shape
    g = make_geom(B, Hh, D, grid)
    d = geom_dims(g)
    topk = int(idx.shape[-1])
    for t, name in ((qc, "qc"), (kc, "kc"), (vc, "vc"), (doc, "doc")):
        _need(t, name, torch.bfloat16, (B, Hh, d.rows, D))
    _need(vt, "vt", torch.bfloat16, (B, Hh, d.n_cubes, D, 64))
    _need(idx, "idx", torch.int32, (B, Hh, d.n_cubes, topk))
    if add is not None:
        for t, name in zip(add, ("dq_add", "dk_add", "dv_add")):
            _need(t, name, torch.bfloat16, (B, Hh, d.rows, D))
    lib = _lib.load()
    nbytes = lib.vsa_linear_bwd_workspace_bytes(g, topk)
    if workspace is None:
        workspace = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=qc.device)
    dq, dk, dv = out if out is not None else (torch.empty_like(qc) for _ in range(3))
    for t, name in ((dq, "dq"), (dk, "dk"), (dv, "dv")):
        _need(t, name, torch.bfloat16, (B, Hh, d.rows, D))
    adds = [t.data_ptr() for t in add] if add is not None else [None, None, None]
    _lib.check("vsa_linear_branch_bwd", lib.vsa_linear_branch_bwd(
        g, qc.data_ptr(), kc.data_ptr(), vc.data_ptr(), vt.data_ptr(), idx.data_ptr(), topk, doc.data_ptr(),
        *adds, dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), workspace.data_ptr(),
        workspace.numel() * workspace.element_size(), _stream()))
    return dq, dk, dv


def mfma_probe(blocks: int, iters: int, device: str = "cuda:0"):
    """Launch the matrix-core probe (vsa_mfma_probe) on the current stream.

    Returns (sink, clk): the fp32 checksums [blocks * 256] and, per workgroup,
    the shader-clock cycles and 100 MHz ticks of its loop (int64 [blocks, 2]).
    Each wavefront issues iters x 8 products of 32768 flops."""
    sink = torch.empty(int(blocks) * 256, dtype=torch.float32, device=device)
    clk = torch.empty((int(blocks), 2), dtype=torch.int64, device=device)
    if not sink.is_cuda:
        raise ValueError("mfma_probe: sink must be on the GPU")
    _lib.check("vsa_mfma_probe", _lib.load().vsa_mfma_probe(int(blocks), int(iters), sink.data_ptr(),
                                                             clk.data_ptr(), _stream()))
    return sink, clk


def sparse_attn_linear_fwd(qc: torch.Tensor, kc: torch.Tensor, vt: torch.Tensor, idx: torch.Tensor,
                           grid: Sequence[int], scale: Optional[float] = None, want_lse: bool = False,
                           out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None):
    """Fine stage and linear branch in one pass: (bf16(O_sparse + O_lin) token-major, lse or None)."""
    B, Hh, Np, D = qc.shape
    g = make_geom(B, Hh, D, grid)
    d = geom_dims(g)
    topk = idx.shape[-1]
    _need(qc, "qc", torch.bfloat16, (B, Hh, d.rows, D))
    _need(kc, "kc", torch.bfloat16, (B, Hh, d.rows, D))
    _need(vt, "vt", torch.bfloat16, (B, Hh, d.n_cubes, D, 64))
    _need(idx, "idx", torch.int32, (B, Hh, d.n_cubes, topk))
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty((B, Hh, d.rows, D), dtype=torch.bfloat16, device=qc.device)
    _need(out, "oc", torch.bfloat16, (B, Hh, d.rows, D))
    lse = torch.empty((B, Hh, d.rows), dtype=torch.float32, device=qc.device) if want_lse else None
    nbytes = workspace_bytes(g, linear=True)
    if workspace is None:
        workspace = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=qc.device)
    _lib.check("vsa_sparse_attn_linear_fwd", _lib.load().vsa_sparse_attn_linear_fwd(
        g, qc.data_ptr(), kc.data_ptr(), vt.data_ptr(), idx.data_ptr(), int(topk), float(scale), out.data_ptr(),
        lse.data_ptr() if lse is not None else None, workspace.data_ptr(),
        workspace.numel() * workspace.element_size(), _stream()))
    return out, lse


class _VsaAttention(torch.autograd.Function):
    """The layer as one autograd node: the forward's kernels, and in backward
    vsa_sparse_attn_bwd (plus vsa_linear_branch_bwd with the fine stage's
    gradients as addends for the hybrid layer) and the unpermutes."""

    @staticmethod
    def forward(ctx, q, k, v, grid, topk, scale, linear, idx):
        qc, qbar = cube_permute_pool(q, grid)
        kc, kbar = cube_permute_pool(k, grid)
        vt = cube_permute(v, grid, layout="dim")
        if idx is None:
            idx = select_topk_pooled(qbar, kbar, grid, topk)
        if linear:
            oc_s, of, lse = sparse_attn_fwd(qc, kc, vt, idx, grid, scale, want_f32=True, want_lse=True)
            oc = linear_branch(qc, kc, vt, idx, of, grid)
        else:
            oc_s, _, lse = sparse_attn_fwd(qc, kc, vt, idx, grid, scale, want_lse=True)
            oc = oc_s
        ctx.save_for_backward(qc, kc, vt, v, oc_s, lse, idx)
        ctx.grid, ctx.scale, ctx.linear = tuple(grid), scale, linear
        ctx.mark_non_differentiable(idx)
        return cube_unpermute(oc, grid), idx

    @staticmethod
    def backward(ctx, do, _unused):
        qc, kc, vt, v, oc_s, lse, idx = ctx.saved_tensors
        grid = ctx.grid
        doc = cube_permute(do.contiguous(), grid)
        vc = cube_permute(v, grid)
        dq, dk, dv = sparse_attn_bwd(qc, kc, vc, oc_s, doc, lse, idx, grid, ctx.scale)
        if ctx.linear:
            dq, dk, dv = linear_branch_bwd(qc, kc, vc, vt, idx, doc, grid, add=(dq, dk, dv), out=(dq, dk, dv))
        return (cube_unpermute(dq, grid), cube_unpermute(dk, grid), cube_unpermute(dv, grid),
                None, None, None, None, None)


def vsa_attention(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, grid: Sequence[int], topk: int,
                  scale: Optional[float] = None, linear: bool = False, idx: Optional[torch.Tensor] = None):
    """One attention layer: [B, S, heads, D] bf16 -> (o [B, S, heads, D] bf16, idx).

    idx: optional block list to use instead of the coarse-stage selection.  When
    gradients are enabled and q, k or v requires them, the layer is one
    autograd node whose backward runs the library's backward kernels.
    """
    if scale is None:
        scale = 1.0 / math.sqrt(q.shape[-1])
    if torch.is_grad_enabled() and (q.requires_grad or k.requires_grad or v.requires_grad):
        return _VsaAttention.apply(q, k, v, grid, topk, scale, linear, idx)
    qc, qbar = cube_permute_pool(q, grid)
    kc, kbar = cube_permute_pool(k, grid)
    vt = cube_permute(v, grid, layout="dim")
    if idx is None:
        idx = select_topk_pooled(qbar, kbar, grid, topk)
    if linear:
        oc, _ = sparse_attn_linear_fwd(qc, kc, vt, idx, grid, scale)
    else:
        oc, _, _ = sparse_attn_fwd(qc, kc, vt, idx, grid, scale)
    return cube_unpermute(oc, grid), idx
