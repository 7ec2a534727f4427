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
    "linear_state",
    "linear_apply",
    "linear_cube_states",
    "linear_unselected",
    "linear_unselected_workspace_bytes",
    "sparse_attn_fwd_linear",
    "sparse_attn_fwd_raster",
    "sparse_attn_fwd_packed",
    "packed_workspace_bytes",
    "sparse_attn_bwd",
    "sparse_attn_linear_fwd",
    "quant_fp8",
    "quant_fp8_workspace_bytes",
    "quant_fp8_noalloc",
    "sparse_attn_fwd_fp8",
    "sparse_attn_fwd_fp8_packed",
    "vsa_attention",
    "workspace_bytes",
    "mfma_probe",
    "hbm_probe",
    "linear_branch_bwd",
    "LayerBuffers",
    "layer_stages",
    "layer_forward",
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


_LAYOUTS = {"token": _lib.VSA_LAYOUT_TOKEN_MAJOR, "dim": _lib.VSA_LAYOUT_DIM_MAJOR,
            "compact": _lib.VSA_LAYOUT_TOKEN_COMPACT, "slots": _lib.VSA_LAYOUT_DIM_SLOTS}


def cube_permute(x: torch.Tensor, grid: Sequence[int], layout: str = "token",
                 out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """[B, S, heads, D] -> cube-major: [B, heads, Np, D] (layout "token", or
    "compact": valid tokens first in each cube), [B, heads, Nc, D, 64] ("dim")
    or [B, heads, Nc, 4, D, 16] ("slots")."""
    B, S, Hh, D = x.shape
    g = make_geom(B, Hh, D, grid)
    d = geom_dims(g)
    _need(x, "x", torch.bfloat16, (B, d.tokens, Hh, D))
    code = _LAYOUTS[layout]
    shape = {"token": (B, Hh, d.rows, D), "compact": (B, Hh, d.rows, D), "dim": (B, Hh, d.n_cubes, D, 64),
             "slots": (B, Hh, d.n_cubes, 4, D, 16)}[layout]
    if out is None:
        out = torch.empty(shape, dtype=torch.bfloat16, device=x.device)
    _need(out, "out", torch.bfloat16, shape)
    _lib.check("vsa_cube_permute",
               _lib.load().vsa_cube_permute(g, x.data_ptr(), out.data_ptr(), code, _stream()))
    return out


def cube_permute_pool(x: torch.Tensor, grid: Sequence[int], out: Optional[torch.Tensor] = None,
                      mean_out: Optional[torch.Tensor] = None, compact: bool = False):
    """Token-major cube permutation and fp32 cube means in one pass: (xc, mean [B, heads, Nc, D]).
    compact: xc in compact order (vsa_cube_permute_pool_compact)."""
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
    fn = "vsa_cube_permute_pool_compact" if compact else "vsa_cube_permute_pool"
    _lib.check(fn, getattr(_lib.load(), fn)(g, x.data_ptr(), out.data_ptr(), mean_out.data_ptr(), _stream()))
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
                           out: Optional[torch.Tensor] = None, out_f32: Optional[torch.Tensor] = None,
                           bf16_out: bool = True):
    """Fine stage on raster-order q and output: returns (o [B, S, heads, D] bf16, lse or None).

    k: raster [B, S, heads, D] (tiles gathered in the kernel) or cube-major [B, heads, Np, D].
    out_f32: optional fp32 output in cube-major rows [B, heads, Np, D] (the
    linear branch's o_sparse); bf16_out=False skips the bf16 output (o is
    then None; out_f32 required).
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
    if bf16_out:
        if out is None:
            out = torch.empty_like(q)
        _need(out, "o", torch.bfloat16, (B, d.tokens, Hh, D))
    else:
        if out_f32 is None:
            raise ValueError("sparse_attn_fwd_raster: bf16_out=False needs out_f32")
        out = None
    if out_f32 is not None:
        _need(out_f32, "o_f32", torch.float32, (B, Hh, d.rows, D))
    lse = torch.empty((B, Hh, d.rows), dtype=torch.float32, device=q.device) if want_lse else None
    _lib.check("vsa_sparse_attn_fwd_raster", _lib.load().vsa_sparse_attn_fwd_raster(
        g, q.data_ptr(), k.data_ptr(), k_layout, vt.data_ptr(), idx.data_ptr(), topk, float(scale),
        out.data_ptr() if out is not None else None, out_f32.data_ptr() if out_f32 is not None else None,
        lse.data_ptr() if lse is not None else None, _stream()))
    return out, lse


def packed_workspace_bytes(g: VsaGeom, topk: int) -> int:
    return int(_lib.load().vsa_sparse_attn_packed_workspace_bytes(g, int(topk)))


def sparse_attn_fwd_packed(q: torch.Tensor, kc: torch.Tensor, vs: torch.Tensor, idx: torch.Tensor,
                           grid: Sequence[int], scale: Optional[float] = None, want_lse: bool = False,
                           out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                           raster: bool = True):
    """Packed fine stage: (o, lse or None).

    q: raster [B, S, heads, D] with o raster (raster=True), or cube-major
    [B, heads, Np, D] with o cube-major (raster=False); kc: compact cube-major
    keys; vs: values in the slot layout [B, heads, Nc, 4, D, 16].
    """
    if raster:
        B, S, Hh, D = q.shape
    else:
        B, Hh, _, D = q.shape
    g = make_geom(B, Hh, D, grid)
    d = geom_dims(g)
    topk = int(idx.shape[-1])
    if raster:
        _need(q, "q", torch.bfloat16, (B, d.tokens, Hh, D))
    else:
        _need(q, "qc", torch.bfloat16, (B, Hh, d.rows, D))
    _need(kc, "kc", torch.bfloat16, (B, Hh, d.rows, D))
    _need(vs, "vs", torch.bfloat16, (B, Hh, d.n_cubes, 4, D, 16))
    _need(idx, "idx", torch.int32, (B, Hh, d.n_cubes, topk))
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty_like(q)
    _need(out, "o", torch.bfloat16, tuple(q.shape))
    lse = torch.empty((B, Hh, d.rows), dtype=torch.float32, device=q.device) if want_lse else None
    nbytes = packed_workspace_bytes(g, topk)
    if workspace is None and nbytes:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=q.device)
    _lib.check("vsa_sparse_attn_fwd_packed", _lib.load().vsa_sparse_attn_fwd_packed(
        g, q.data_ptr(), _lib.VSA_LAYOUT_RASTER if raster else _lib.VSA_LAYOUT_TOKEN_MAJOR, kc.data_ptr(),
        vs.data_ptr(), idx.data_ptr(), topk, float(scale), out.data_ptr(),
        lse.data_ptr() if lse is not None else None,
        workspace.data_ptr() if workspace is not None else None,
        workspace.numel() * workspace.element_size() if workspace is not None else 0, _stream()))
    return out, lse


def quant_fp8_workspace_bytes(g: VsaGeom) -> int:
    return int(_lib.load().vsa_quant_fp8_workspace_bytes(g))


def quant_fp8(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, grid: Sequence[int], want_means: bool = False,
              out=None, workspace: Optional[torch.Tensor] = None, noalloc: bool = False, packed: bool = False):
    """E4M3 codes of raster Q, K (per (b, h, cube)) and V (per (b, h, channel)).

    Returns (q8, qscale, k8, kscale, v8t, vscale, qmean, kmean): codes uint8
    [B, heads, Np, D] and [B, heads, Nc, D, 64], scales f32 [B, heads, Nc] and
    [B, heads, D], cube means f32 [B, heads, Nc, D] or None.  `out`: optional
    tuple of the same eight tensors to write into (means may be None).
    noalloc: use vsa_quant_fp8_noalloc (the library's static scratch instead
    of a workspace; with `out` given, nothing is allocated).
    packed: vsa_quant_fp8_packed, the layouts of the packed fp8 stage: K codes
    in compact cube-major rows, V codes [B, heads, Nc, 4, D, 16] (slots).
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
               torch.empty((B, Hh, d.n_cubes, 4, D, 16) if packed else (B, Hh, d.n_cubes, D, 64), **u8),
               torch.empty((B, Hh, D), **f32),
               torch.empty((B, Hh, d.n_cubes, D), **f32) if want_means else None,
               torch.empty((B, Hh, d.n_cubes, D), **f32) if want_means else None)
    q8, qs, k8, ks, v8t, vs, qm, km = out
    _need(q8, "q8", torch.uint8, (B, Hh, d.rows, D))
    _need(k8, "k8", torch.uint8, (B, Hh, d.rows, D))
    _need(v8t, "v8s" if packed else "v8t", torch.uint8,
          (B, Hh, d.n_cubes, 4, D, 16) if packed else (B, Hh, d.n_cubes, D, 64))
    _need(qs, "qscale", torch.float32, (B, Hh, d.n_cubes))
    _need(ks, "kscale", torch.float32, (B, Hh, d.n_cubes))
    _need(vs, "vscale", torch.float32, (B, Hh, D))
    for t, n in ((qm, "qmean"), (km, "kmean")):
        if t is not None:
            _need(t, n, torch.float32, (B, Hh, d.n_cubes, D))
    lib = _lib.load()
    if noalloc and packed:
        raise ValueError("quant_fp8: the allocation-free entry point writes the unpacked layouts only")
    if noalloc:
        _lib.check("vsa_quant_fp8_noalloc", lib.vsa_quant_fp8_noalloc(
            g, q.data_ptr(), k.data_ptr(), v.data_ptr(), q8.data_ptr(), qs.data_ptr(), k8.data_ptr(),
            ks.data_ptr(), v8t.data_ptr(), vs.data_ptr(), qm.data_ptr() if qm is not None else None,
            km.data_ptr() if km is not None else None, _stream()))
        return q8, qs, k8, ks, v8t, vs, qm, km
    nbytes = lib.vsa_quant_fp8_workspace_bytes(g)
    if workspace is None:
        workspace = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=dev)
    fn = "vsa_quant_fp8_packed" if packed else "vsa_quant_fp8"
    _lib.check(fn, getattr(lib, fn)(
        g, q.data_ptr(), k.data_ptr(), v.data_ptr(), q8.data_ptr(), qs.data_ptr(), k8.data_ptr(), ks.data_ptr(),
        v8t.data_ptr(), vs.data_ptr(), qm.data_ptr() if qm is not None else None,
        km.data_ptr() if km is not None else None, workspace.data_ptr(),
        workspace.numel() * workspace.element_size(), _stream()))
    return q8, qs, k8, ks, v8t, vs, qm, km


def quant_fp8_noalloc(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, grid: Sequence[int],
                      want_means: bool = False, out=None):
    """quant_fp8 through vsa_quant_fp8_noalloc (no workspace; see include/vsa_cube.h)."""
    return quant_fp8(q, k, v, grid, want_means=want_means, out=out, noalloc=True)


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


def sparse_attn_fwd_fp8_packed(q8: torch.Tensor, qscale: torch.Tensor, k8c: torch.Tensor, kscale: torch.Tensor,
                               v8s: torch.Tensor, vscale: torch.Tensor, idx: torch.Tensor, grid: Sequence[int],
                               scale: Optional[float] = None, want_lse: bool = False,
                               out: Optional[torch.Tensor] = None, raster: bool = False,
                               workspace: Optional[torch.Tensor] = None):
    """fp8 fine stage on packed tiles (vsa_sparse_attn_fwd_fp8_packed), on the
    layouts of quant_fp8(packed=True).  Returns (o bf16, lse or None) as
    sparse_attn_fwd_fp8.  workspace: the packing plan (packed_workspace_bytes)."""
    B, Hh, Np, D = q8.shape
    g = make_geom(B, Hh, D, grid)
    d = geom_dims(g)
    topk = int(idx.shape[-1])
    _need(q8, "q8", torch.uint8, (B, Hh, d.rows, D))
    _need(k8c, "k8c", torch.uint8, (B, Hh, d.rows, D))
    _need(v8s, "v8s", torch.uint8, (B, Hh, d.n_cubes, 4, D, 16))
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
    nbytes = packed_workspace_bytes(g, topk)
    if workspace is None and nbytes:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=q8.device)
    layout = _lib.VSA_LAYOUT_RASTER if raster else _lib.VSA_LAYOUT_TOKEN_MAJOR
    _lib.check("vsa_sparse_attn_fwd_fp8_packed", _lib.load().vsa_sparse_attn_fwd_fp8_packed(
        g, q8.data_ptr(), qscale.data_ptr(), k8c.data_ptr(), kscale.data_ptr(), v8s.data_ptr(), vscale.data_ptr(),
        idx.data_ptr(), topk, float(scale), layout, out.data_ptr(), lse.data_ptr() if lse is not None else None,
        workspace.data_ptr() if workspace is not None else None,
        workspace.numel() * workspace.element_size() if workspace is not None else 0, _stream()))
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
                  workspace: Optional[torch.Tensor] = None, save: bool = False, raster: bool = False):
    """bf16(o_sparse + O_lin), token-major.

    save: also return (o_lin fp32 [B, heads, Np, D], inv_den fp32 [B, heads, Np]) for
    linear_branch_bwd(saved=...): (out, (o_lin, inv_den)).
    raster: qc is the raster queries [B, S, heads, D] and the output is raster
    [B, S, heads, D] (kc, vt, o_sparse and the saved values stay cube-major).
    """
    B, Hh, D = kc.shape[0], kc.shape[1], kc.shape[3]
    g = make_geom(B, Hh, D, grid)
    d = geom_dims(g)
    topk = idx.shape[-1]
    qo_shape = (B, d.tokens, Hh, D) if raster else (B, Hh, d.rows, D)
    _need(qc, "q" if raster else "qc", torch.bfloat16, qo_shape)
    _need(kc, "kc", torch.bfloat16, (B, Hh, d.rows, D))
    _need(vt, "vt", torch.bfloat16, (B, Hh, d.n_cubes, D, 64))
    _need(idx, "idx", torch.int32, (B, Hh, d.n_cubes, topk))
    _need(o_sparse, "o_sparse", torch.float32, (B, Hh, d.rows, D))
    if out is None:
        out = torch.empty(qo_shape, dtype=torch.bfloat16, device=qc.device)
    _need(out, "o" if raster else "oc", torch.bfloat16, qo_shape)
    nbytes = workspace_bytes(g, linear=True)
    if workspace is None:
        workspace = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=qc.device)
    o_lin = inv_den = None
    if save:
        o_lin = torch.empty((B, Hh, d.rows, D), dtype=torch.float32, device=qc.device)
        inv_den = torch.empty((B, Hh, d.rows), dtype=torch.float32, device=qc.device)
    _lib.check("vsa_linear_branch", _lib.load().vsa_linear_branch(
        g, qc.data_ptr(), _lib.VSA_LAYOUT_RASTER if raster else _lib.VSA_LAYOUT_TOKEN_MAJOR, kc.data_ptr(),
        vt.data_ptr(), idx.data_ptr(), int(topk), o_sparse.data_ptr(),
        out.data_ptr(), o_lin.data_ptr() if save else None, inv_den.data_ptr() if save else None,
        workspace.data_ptr(), workspace.numel() * workspace.element_size(), _stream()))
    return (out, (o_lin, inv_den)) if save else out


def linear_state(kc: torch.Tensor, vt: torch.Tensor, grid: Sequence[int], workspace: torch.Tensor) -> None:
    """The linear branch's state pass (vsa_linear_state): phi(K), S_tot and z_tot into `workspace`."""
    B, Hh, _, D = kc.shape
    g = make_geom(B, Hh, D, grid)
    d = geom_dims(g)
    _need(kc, "kc", torch.bfloat16, (B, Hh, d.rows, D))
    _need(vt, "vt", torch.bfloat16, (B, Hh, d.n_cubes, D, 64))
    _lib.check("vsa_linear_state", _lib.load().vsa_linear_state(
        g, kc.data_ptr(), vt.data_ptr(), workspace.data_ptr(), workspace.numel() * workspace.element_size(),
        _stream()))


def linear_apply(q: torch.Tensor, vt: torch.Tensor, idx: torch.Tensor, o_sparse: torch.Tensor,
                 grid: Sequence[int], workspace: torch.Tensor, out: Optional[torch.Tensor] = None,
                 raster: bool = False):
    """The rest of linear_branch (vsa_linear_apply) on a workspace that
    linear_state filled for the same keys and values: bf16(o_sparse + O_lin),
    raster (q and output [B, S, heads, D]) or token-major."""
    B, Hh, D = vt.shape[0], vt.shape[1], vt.shape[3]
    g = make_geom(B, Hh, D, grid)
    d = geom_dims(g)
    topk = idx.shape[-1]
    qo_shape = (B, d.tokens, Hh, D) if raster else (B, Hh, d.rows, D)
    _need(q, "q" if raster else "qc", torch.bfloat16, qo_shape)
    _need(vt, "vt", torch.bfloat16, (B, Hh, d.n_cubes, D, 64))
    _need(idx, "idx", torch.int32, (B, Hh, d.n_cubes, topk))
    _need(o_sparse, "o_sparse", torch.float32, (B, Hh, d.rows, D))
    if out is None:
        out = torch.empty(qo_shape, dtype=torch.bfloat16, device=q.device)
    _need(out, "o" if raster else "oc", torch.bfloat16, qo_shape)
    _lib.check("vsa_linear_apply", _lib.load().vsa_linear_apply(
        g, q.data_ptr(), _lib.VSA_LAYOUT_RASTER if raster else _lib.VSA_LAYOUT_TOKEN_MAJOR, vt.data_ptr(),
        idx.data_ptr(), int(topk), o_sparse.data_ptr(), out.data_ptr(), None, None, workspace.data_ptr(),
        workspace.numel() * workspace.element_size(), _stream()))
    return out


def linear_cube_states(kc: torch.Tensor, vt: torch.Tensor, grid: Sequence[int],
                       out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Per-cube states of the linear branch (vsa_linear_cube_states): bf16
    [B, heads, D + 1, Nc, D], [.., e, j, d] = (phi(K_j)^T V_j)[d, e] for e < D
    and the column sums of phi(K_j) at e = D."""
    B, Hh, _, D = kc.shape
    g = make_geom(B, Hh, D, grid)
    d = geom_dims(g)
    _need(kc, "kc", torch.bfloat16, (B, Hh, d.rows, D))
    _need(vt, "vt", torch.bfloat16, (B, Hh, d.n_cubes, D, 64))
    shape = (B, Hh, D + 1, d.n_cubes, D)
    if out is None:
        out = torch.empty(shape, dtype=torch.bfloat16, device=kc.device)
    _need(out, "states", torch.bfloat16, shape)
    _lib.check("vsa_linear_cube_states", _lib.load().vsa_linear_cube_states(
        g, kc.data_ptr(), vt.data_ptr(), out.data_ptr(), _stream()))
    return out


def linear_unselected_workspace_bytes(g: VsaGeom) -> int:
    return int(_lib.load().vsa_linear_unselected_workspace_bytes(g))


def linear_unselected(states: torch.Tensor, idx: torch.Tensor, grid: Sequence[int],
                      out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Summed states of every query cube's unselected key cubes
    (vsa_linear_unselected): bf16 [B, heads, Nc, D * D + D], S_U^T rows then z_U."""
    B, Hh, D = states.shape[0], states.shape[1], states.shape[4]
    g = make_geom(B, Hh, D, grid)
    d = geom_dims(g)
    topk = idx.shape[-1]
    _need(states, "states", torch.bfloat16, (B, Hh, D + 1, d.n_cubes, D))
    _need(idx, "idx", torch.int32, (B, Hh, d.n_cubes, topk))
    shape = (B, Hh, d.n_cubes, D * D + D)
    if out is None:
        out = torch.empty(shape, dtype=torch.bfloat16, device=states.device)
    _need(out, "su", torch.bfloat16, shape)
    if workspace is None:
        workspace = torch.empty(max(16, linear_unselected_workspace_bytes(g)), dtype=torch.uint8,
                                device=states.device)
    _lib.check("vsa_linear_unselected", _lib.load().vsa_linear_unselected(
        g, states.data_ptr(), idx.data_ptr(), int(topk), out.data_ptr(), workspace.data_ptr(),
        workspace.numel() * workspace.element_size(), _stream()))
    return out


def sparse_attn_fwd_linear(q: torch.Tensor, kc: torch.Tensor, vt: torch.Tensor, idx: torch.Tensor,
                           su: torch.Tensor, grid: Sequence[int], scale: Optional[float] = None,
                           raster: bool = True, out: Optional[torch.Tensor] = None,
                           lse: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Fine stage plus the linear branch from summed states
    (vsa_sparse_attn_fwd_linear): bf16(O_sparse + phi(Q) S_U / (phi(Q) . z_U)),
    q and the output raster [B, S, heads, D] (or cube-major rows)."""
    B, Hh, _, D = kc.shape
    g = make_geom(B, Hh, D, grid)
    d = geom_dims(g)
    topk = idx.shape[-1]
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    qo_shape = (B, d.tokens, Hh, D) if raster else (B, Hh, d.rows, D)
    _need(q, "q" if raster else "qc", torch.bfloat16, qo_shape)
    _need(kc, "kc", torch.bfloat16, (B, Hh, d.rows, D))
    _need(vt, "vt", torch.bfloat16, (B, Hh, d.n_cubes, D, 64))
    _need(idx, "idx", torch.int32, (B, Hh, d.n_cubes, topk))
    _need(su, "su", torch.bfloat16, (B, Hh, d.n_cubes, D * D + D))
    if out is None:
        out = torch.empty(qo_shape, dtype=torch.bfloat16, device=q.device)
    _need(out, "o", torch.bfloat16, qo_shape)
    if lse is not None:
        _need(lse, "lse", torch.float32, (B, Hh, d.rows))
    _lib.check("vsa_sparse_attn_fwd_linear", _lib.load().vsa_sparse_attn_fwd_linear(
        g, q.data_ptr(), _lib.VSA_LAYOUT_RASTER if raster else _lib.VSA_LAYOUT_TOKEN_MAJOR, kc.data_ptr(),
        vt.data_ptr(), idx.data_ptr(), int(topk), float(scale), su.data_ptr(), out.data_ptr(),
        lse.data_ptr() if lse is not None else None, _stream()))
    return out


def linear_branch_bwd(qc: torch.Tensor, kc: torch.Tensor, vc: torch.Tensor, vt: torch.Tensor, idx: torch.Tensor,
                      doc: torch.Tensor, grid: Sequence[int], workspace: Optional[torch.Tensor] = None,
                      add: Optional[Tuple[torch.Tensor, torch.Tensor, torch.Tensor]] = None, out=None,
                      saved: Optional[Tuple[torch.Tensor, torch.Tensor]] = None):
    """Gradients of the linear branch.  Returns (dq, dk, dv), bf16 [B, heads, Np, D] token-major.

    qc, kc, vc, doc: Q, K, V and dO token-major; vt: V DIM_MAJOR; idx: the block lists.
    add: optional (dq, dk, dv) added before the one bf16 rounding (the fine stage's, for the
    hybrid layer); out: optional output tensors (may be the addends themselves).
    saved: optional (o_lin, inv_den) from linear_branch(save=True) on the same inputs.
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
    sv = [None, None]
    if saved is not None:
        _need(saved[0], "o_lin", torch.float32, (B, Hh, d.rows, D))
        _need(saved[1], "inv_den", torch.float32, (B, Hh, d.rows))
        sv = [saved[0].data_ptr(), saved[1].data_ptr()]
    _lib.check("vsa_linear_branch_bwd", lib.vsa_linear_branch_bwd(
        g, qc.data_ptr(), kc.data_ptr(), vc.data_ptr(), vt.data_ptr(), idx.data_ptr(), topk, doc.data_ptr(),
        *sv, *adds, dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), workspace.data_ptr(),
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


def hbm_probe(kind: str, src: Optional[torch.Tensor], dst: Optional[torch.Tensor]) -> None:
    """Launch one HBM stream (vsa_hbm_probe) on the current stream: kind
    "copy" (src -> dst, equal byte sizes), "read" (src) or "write" (dst)."""
    code = {"copy": 0, "read": 1, "write": 2}[kind]
    t = src if src is not None else dst
    nbytes = t.numel() * t.element_size()
    for x in (src, dst):
        if x is not None and (not x.is_cuda or not x.is_contiguous()):
            raise ValueError("hbm_probe: buffers must be contiguous GPU tensors")
    if kind == "copy" and dst.numel() * dst.element_size() != nbytes:
        raise ValueError("hbm_probe: copy buffers differ in size")
    _lib.check("vsa_hbm_probe", _lib.load().vsa_hbm_probe(code, src.data_ptr() if src is not None else None,
                                                           dst.data_ptr() if dst is not None else None, nbytes,
                                                           _stream()))


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
        o_lin = inv_den = None
        if linear:
            oc_s, of, lse = sparse_attn_fwd(qc, kc, vt, idx, grid, scale, want_f32=True, want_lse=True)
            oc, (o_lin, inv_den) = linear_branch(qc, kc, vt, idx, of, grid, save=True)
        else:
            oc_s, _, lse = sparse_attn_fwd(qc, kc, vt, idx, grid, scale, want_lse=True)
            oc = oc_s
        ctx.save_for_backward(qc, kc, vt, v, oc_s, lse, idx, o_lin, inv_den)
        ctx.grid, ctx.scale, ctx.linear = tuple(grid), scale, linear
        ctx.mark_non_differentiable(idx)
        return cube_unpermute(oc, grid), idx

    @staticmethod
    def backward(ctx, do, _unused):
        qc, kc, vt, v, oc_s, lse, idx, o_lin, inv_den = ctx.saved_tensors
        grid = ctx.grid
        doc = cube_permute(do.contiguous(), grid)
        vc = cube_permute(v, grid)
        dq, dk, dv = sparse_attn_bwd(qc, kc, vc, oc_s, doc, lse, idx, grid, ctx.scale)
        if ctx.linear:
            dq, dk, dv = linear_branch_bwd(qc, kc, vc, vt, idx, doc, grid, add=(dq, dk, dv), out=(dq, dk, dv),
                                           saved=(o_lin, inv_den))
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


class LayerBuffers:
    """Device tensors of one forward layer (layer_forward), allocated once so
    that repeated layers allocate nothing."""

    def __init__(self, batch: int, heads: int, head_dim: int, grid: Sequence[int], topk: int,
                 linear: bool = False, device="cuda:0"):
        B, H, D = int(batch), int(heads), int(head_dim)
        self.geom = g = make_geom(B, H, D, grid)
        d = geom_dims(g)
        dev = torch.device(device)
        self.qc = torch.empty((B, H, d.rows, D), dtype=torch.bfloat16, device=dev)
        self.kc = torch.empty_like(self.qc)
        self.vt = torch.empty((B, H, d.n_cubes, D, 64), dtype=torch.bfloat16, device=dev)
        self.qbar = torch.empty((B, H, d.n_cubes, D), dtype=torch.float32, device=dev)
        self.kbar = torch.empty_like(self.qbar)
        self.idx = torch.empty((B, H, d.n_cubes, int(topk)), dtype=torch.int32, device=dev)
        self.ws_sel = torch.empty(max(16, workspace_bytes(g)), dtype=torch.uint8, device=dev)
        # Packed fine stage: V in the slot layout and the packing plan.
        self.vs = torch.empty((B, H, d.n_cubes, 4, D, 16), dtype=torch.bfloat16, device=dev)
        nplan = packed_workspace_bytes(g, topk)
        self.ws_plan = torch.empty(nplan, dtype=torch.uint8, device=dev) if nplan else None
        self.oc = torch.empty_like(self.qc) if linear else None
        self.oc2 = torch.empty_like(self.qc) if linear else None
        self.of = torch.empty((B, H, d.rows, D), dtype=torch.float32, device=dev) if linear else None
        self.ws_lin = (torch.empty(max(16, workspace_bytes(g, linear=True)), dtype=torch.uint8, device=dev)
                       if linear else None)
        # Linear branch from summed states: per-cube states, summed states per
        # query cube and the selection bits.
        self.states = (torch.empty((B, H, D + 1, d.n_cubes, D), dtype=torch.bfloat16, device=dev)
                       if linear else None)
        self.su = torch.empty((B, H, d.n_cubes, D * D + D), dtype=torch.bfloat16, device=dev) if linear else None
        self.ws_bits = (torch.empty(max(16, linear_unselected_workspace_bytes(g)), dtype=torch.uint8, device=dev)
                        if linear else None)
        # Second stream (default priority) for the V permute, which depends on
        # nothing the coarse stage makes and runs beside it.
        self.side = torch.cuda.Stream(device=dev)
        # Recorded on the side stream after the V permute and after the
        # linear state pass; the caller's stream waits for each where needed.
        self.ev_v = torch.cuda.Event()
        self.ev_state = torch.cuda.Event()


def layer_stages(linear: bool = False, fused_linear: bool = False, linear_mode: str = "states"):
    """Names of the stages layer_forward runs, in order (its `mark` hook is
    called once before the first and once after each)."""
    if linear:
        if fused_linear:
            return ["permute", "select", "fine+linear", "unpermute"]
        if linear_mode == "states":
            return ["pool", "select", "unselected", "fine+linear"]
        return ["pool", "select", "fine", "linear"]
    return ["pool", "select", "fine"]


def layer_forward(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, grid: Sequence[int], topk: int,
                  scale: Optional[float] = None, linear: bool = False, fused_linear: bool = False,
                  k_raster: bool = False, window: Optional[Sequence[int]] = None,
                  bufs: Optional[LayerBuffers] = None, out: Optional[torch.Tensor] = None, mark=None,
                  packed: bool = True, overlap: bool = True, linear_mode: str = "states"):
    """One forward attention layer on raster q, k, v [B, S, heads, D] bf16:
    returns (o [B, S, heads, D] bf16, idx).

    Without the linear branch the fine stage reads Q and writes O in raster
    order: Q is only pooled, K is pooled and permuted in one pass, V is
    permuted; with `packed` (the default) and a grid with partial cubes, K in
    compact order, V in the slot layout and the packed fine stage (edge cubes
    share tiles), otherwise K
    token-major (or, with k_raster, only pooled and its tiles gathered by the
    fine stage), V cube-transposed and the unpacked stage.  window: a sliding-tile window
    (cubes per axis) whose static block lists replace the coarse stage.  The
    hybrid layer (linear branch) permutes K into cube-major rows (the branch's
    state reads them).  With two calls, the fine stage and the linear branch
    both read raster Q and the branch writes the raster output, so Q is only
    pooled; the fused pass (fused_linear) permutes Q too and unpermutes.  mark(i), if given, is called before
    stage 0 and after each stage i - 1 (layer_stages names them).

    Streams: the V permute runs on a second stream (bufs.side) after the Q and
    K pooling, beside the coarse stage (selection: matrix cores and lane
    arithmetic; the permute: memory traffic); the caller's stream waits for it
    before the fine stage.  In the hybrid two-call layer the linear branch's
    state pass follows it there, beside the coarse and fine stages, and the
    caller's stream waits for it before the rest of the branch.  The layer is
    thus ordered on the caller's stream as a whole.  The stage marks are taken on the caller's stream (the select stage
    ends once the permute has too).  overlap=False keeps every launch on the
    caller's stream (for per-kernel timings that no other kernel shares).
    """
    B, S, H, D = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if linear_mode not in ("states", "tiles"):
        raise ValueError(f"linear_mode must be 'states' or 'tiles', not {linear_mode!r}")
    states_mode = linear and not fused_linear and linear_mode == "states"
    if bufs is None:
        bufs = LayerBuffers(B, H, D, grid, topk, linear=linear, device=q.device)
    if out is None:
        out = torch.empty_like(q)
    mark = mark or (lambda i: None)
    b = bufs
    mark(0)
    # Packing pays only where cubes hold padding; on other grids the packed
    # stage is the unpacked one with another V layout (and slightly slower).
    packed = packed and not k_raster and any(int(x) % 4 for x in grid)
    if linear:
        # Two calls: both read raster Q and the linear branch writes the raster
        # output, so Q is only pooled.  The fused pass works on cube-major Q.
        if fused_linear:
            cube_permute_pool(q, grid, out=b.qc, mean_out=b.qbar)
        else:
            cube_pool(q, grid, mean_out=b.qbar)
        cube_permute_pool(k, grid, out=b.kc, mean_out=b.kbar)
    elif window is None:
        cube_pool(q, grid, mean_out=b.qbar)
        if k_raster:
            cube_pool(k, grid, mean_out=b.kbar)
        else:
            cube_permute_pool(k, grid, out=b.kc, mean_out=b.kbar, compact=packed)
    elif not k_raster:
        cube_permute(k, grid, layout="compact" if packed else "token", out=b.kc)
    main = torch.cuda.current_stream(q.device)
    side = b.side if overlap else main
    # The side stream starts once the pooling is queued (and so after the
    # previous layer's reads of the V buffer on the caller's stream).
    side.wait_stream(main)
    with torch.cuda.stream(side):
        if packed and not linear:
            cube_permute(v, grid, layout="slots", out=b.vs)
        else:
            cube_permute(v, grid, layout="dim", out=b.vt)
        b.ev_v.record(side)
        if states_mode:
            # The per-cube states need only K and V: they run here too, beside
            # the coarse stage.
            linear_cube_states(b.kc, b.vt, grid, out=b.states)
            b.ev_state.record(side)
        elif linear and not fused_linear:
            # The linear branch's state (phi(K), S_tot, z_tot) needs only K and
            # V: it runs here too, beside the coarse and fine stages.
            linear_state(b.kc, b.vt, grid, b.ws_lin)
            b.ev_state.record(side)
    mark(1)
    if window is not None:
        # The sliding-tile list is static; it is rebuilt every layer all the same.
        sta_index(grid, window, B, H, head_dim=D, out=b.idx)
    else:
        select_topk_pooled(b.qbar, b.kbar, grid, topk, out=b.idx, workspace=b.ws_sel)
    main.wait_event(b.ev_v)
    mark(2)
    if not linear:
        if packed:
            sparse_attn_fwd_packed(q, b.kc, b.vs, b.idx, grid, scale, out=out, workspace=b.ws_plan)
        else:
            sparse_attn_fwd_raster(q, k if k_raster else b.kc, b.vt, b.idx, grid, scale, out=out)
        mark(3)
        return out, b.idx
    if states_mode:
        # The summed states of every query cube's unselected cubes, then the
        # fine stage, which adds the linear branch in its epilogue.
        main.wait_event(b.ev_state)
        linear_unselected(b.states, b.idx, grid, out=b.su, workspace=b.ws_bits)
        mark(3)
        sparse_attn_fwd_linear(q, b.kc, b.vt, b.idx, b.su, grid, scale, raster=True, out=out)
        mark(4)
        return out, b.idx
    if fused_linear:
        sparse_attn_linear_fwd(b.qc, b.kc, b.vt, b.idx, grid, scale, out=b.oc2, workspace=b.ws_lin)
        mark(3)
        cube_unpermute(b.oc2, grid, out=out)
        mark(4)
        return out, b.idx
    sparse_attn_fwd_raster(q, b.kc, b.vt, b.idx, grid, scale, out_f32=b.of, bf16_out=False)
    mark(3)
    main.wait_event(b.ev_state)
    linear_apply(q, b.vt, b.idx, b.of, grid, b.ws_lin, out=out, raster=True)
    mark(4)
    return out, b.idx
