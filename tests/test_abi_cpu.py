"""C ABI checks that need no GPU: the library loads, exports every function the
header declares, and host-side validation returns the documented status before
anything is launched (only invalid arguments are passed, so no kernel runs)."""

import ctypes
import os
import re

import pytest

import workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "vsa_cube.h")


def header_functions():
    text = open(HEADER, encoding="utf-8").read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(vsa_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    from block_sparse_video_cube_amd import _lib

    if not os.path.exists(_lib.LIB_PATH):
        pytest.fail("libvsa_cube.so is not built (run __graft_entry__.build())")
    return _lib.load()


def test_header_and_binding_agree():
    from block_sparse_video_cube_amd import _lib

    assert header_functions() == sorted(_lib.ENTRY_POINTS)


def test_every_declared_symbol_is_exported(lib):
    for name in header_functions():
        assert hasattr(lib, name), name


def test_abi_version_and_status_text(lib):
    assert lib.vsa_abi_version() == 4
    for code in range(12):
        assert lib.vsa_status_string(code)
    assert lib.vsa_status_string(12345) == b"unknown status"


def geom(B=1, H=2, D=64, grid=(8, 8, 8)):
    from block_sparse_video_cube_amd import make_geom

    return make_geom(B, H, D, grid)


@pytest.mark.parametrize("name", list(workloads.WORKLOADS))
def test_geom_dims_match_workloads(lib, name):
    from block_sparse_video_cube_amd import _lib

    wl = workloads.workload(name)
    d = _lib.VsaDims()
    assert lib.vsa_geom_dims(geom(wl.batch, wl.heads, wl.head_dim, wl.grid), ctypes.byref(d)) == 0
    assert (d.pad_t, d.pad_h, d.pad_w) == wl.padded_grid
    assert d.n_cubes == wl.n_cubes
    assert d.tokens == wl.tokens
    assert d.rows == wl.rows


def test_geom_errors(lib):
    from block_sparse_video_cube_amd import _lib

    d = _lib.VsaDims()
    assert lib.vsa_geom_dims(None, ctypes.byref(d)) == _lib.VSA_ERR_NULL
    assert lib.vsa_geom_dims(geom(), None) == _lib.VSA_ERR_NULL
    assert lib.vsa_geom_dims(geom(B=0), ctypes.byref(d)) == _lib.VSA_ERR_GEOMETRY
    assert lib.vsa_geom_dims(geom(grid=(0, 4, 4)), ctypes.byref(d)) == _lib.VSA_ERR_GEOMETRY
    assert lib.vsa_geom_dims(geom(H=-3), ctypes.byref(d)) == _lib.VSA_ERR_GEOMETRY
    assert lib.vsa_geom_dims(geom(D=96), ctypes.byref(d)) == _lib.VSA_ERR_HEAD_DIM
    assert lib.vsa_geom_dims(geom(B=300, H=300), ctypes.byref(d)) == _lib.VSA_ERR_GEOMETRY


def test_workspace_sizes(lib):
    g = geom()
    assert lib.vsa_select_workspace_bytes(g) >= 2 * 2 * 8 * 64 * 4
    assert lib.vsa_linear_workspace_bytes(g) >= 2 * 512 * 64 * 2
    assert lib.vsa_select_workspace_bytes(geom(D=65)) == 0
    assert lib.vsa_linear_workspace_bytes(geom(B=0)) == 0


FAKE = 0x10000  # 16-byte aligned, never dereferenced: validation fails first
ODD = 0x10008   # 8-byte aligned only


def test_entry_points_reject_bad_arguments_before_launch(lib):
    from block_sparse_video_cube_amd import _lib

    g = geom()
    P = FAKE
    # Permute / unpermute.
    assert lib.vsa_cube_permute(g, None, P, 0, None) == _lib.VSA_ERR_NULL
    assert lib.vsa_cube_permute(g, P, ODD, 0, None) == _lib.VSA_ERR_ALIGN
    assert lib.vsa_cube_permute(g, P, P, 7, None) == _lib.VSA_ERR_LAYOUT
    assert lib.vsa_cube_permute(geom(D=32), P, P, 0, None) == _lib.VSA_ERR_HEAD_DIM
    assert lib.vsa_cube_unpermute(g, P, None, None) == _lib.VSA_ERR_NULL
    assert lib.vsa_cube_unpermute(geom(grid=(1, 0, 1)), P, P, None) == _lib.VSA_ERR_GEOMETRY
    # Select.
    ws = lib.vsa_select_workspace_bytes(g)
    assert lib.vsa_select_topk(g, P, P, 2, P, None, ws, None) == _lib.VSA_ERR_NULL
    assert lib.vsa_select_topk(g, P, P, 0, P, P, ws, None) == _lib.VSA_ERR_TOPK
    assert lib.vsa_select_topk(g, P, P, 9, P, P, ws, None) == _lib.VSA_ERR_TOPK
    assert lib.vsa_select_topk(g, P, P, 2, P, P, ws - 1, None) == _lib.VSA_ERR_WORKSPACE
    assert lib.vsa_select_topk(g, P, ODD, 2, P, P, ws, None) == _lib.VSA_ERR_ALIGN
    big = geom(grid=(4 * 17, 4 * 16, 4 * 16))  # 4352 cubes > VSA_MAX_CUBES
    assert lib.vsa_select_topk(big, P, P, 2, P, P, 1 << 40, None) == _lib.VSA_ERR_GEOMETRY
    # Fine stage.
    assert lib.vsa_sparse_attn_fwd(g, P, P, P, None, 2, 0.125, P, None, None, None) == _lib.VSA_ERR_NULL
    assert lib.vsa_sparse_attn_fwd(g, P, P, P, P, 0, 0.125, P, None, None, None) == _lib.VSA_ERR_TOPK
    assert lib.vsa_sparse_attn_fwd(g, P, P, P, P, 2, 0.0, P, None, None, None) == _lib.VSA_ERR_SCALE
    assert lib.vsa_sparse_attn_fwd(g, P, P, P, P, 2, float("nan"), P, None, None, None) == _lib.VSA_ERR_SCALE
    assert lib.vsa_sparse_attn_fwd(g, P, P, P, P, 2, float("inf"), P, None, None, None) == _lib.VSA_ERR_SCALE
    assert lib.vsa_sparse_attn_fwd(g, P, P, P, P, 2, 0.125, P, ODD, None, None) == _lib.VSA_ERR_ALIGN
    # Linear branch.
    lws = lib.vsa_linear_workspace_bytes(g)
    assert lib.vsa_linear_branch(g, P, 0, P, P, P, 2, None, P, None, None, P, lws, None) == _lib.VSA_ERR_NULL
    assert lib.vsa_linear_branch(g, P, 0, P, P, P, 2, P, P, None, None, P, lws - 1, None) == _lib.VSA_ERR_WORKSPACE
    assert lib.vsa_linear_branch(g, P, 0, P, P, P, 99, P, P, None, None, P, lws, None) == _lib.VSA_ERR_TOPK
    # The saved O_lin and 1/den come as a pair, 16-byte aligned.
    assert lib.vsa_linear_branch(g, P, 0, P, P, P, 2, P, P, P, None, P, lws, None) == _lib.VSA_ERR_NULL
    assert lib.vsa_linear_branch(g, P, 0, P, P, P, 2, P, P, None, P, P, lws, None) == _lib.VSA_ERR_NULL
    assert lib.vsa_linear_branch(g, P, 0, P, P, P, 2, P, P, ODD, P, P, lws, None) == _lib.VSA_ERR_ALIGN
    # The branch in two parts.
    assert lib.vsa_linear_state(g, None, P, P, lws, None) == _lib.VSA_ERR_NULL
    assert lib.vsa_linear_state(g, P, ODD, P, lws, None) == _lib.VSA_ERR_ALIGN
    assert lib.vsa_linear_state(g, P, P, P, lws - 1, None) == _lib.VSA_ERR_WORKSPACE
    assert lib.vsa_linear_state(geom(D=32), P, P, P, lws, None) == _lib.VSA_ERR_HEAD_DIM
    assert lib.vsa_linear_apply(g, P, 0, P, P, 2, None, P, None, None, P, lws, None) == _lib.VSA_ERR_NULL
    assert lib.vsa_linear_apply(g, P, 0, P, P, 2, P, P, P, None, P, lws, None) == _lib.VSA_ERR_NULL
    assert lib.vsa_linear_apply(g, P, 0, P, P, 2, P, ODD, None, None, P, lws, None) == _lib.VSA_ERR_ALIGN
    assert lib.vsa_linear_apply(g, P, 0, P, P, 0, P, P, None, None, P, lws, None) == _lib.VSA_ERR_TOPK
    assert lib.vsa_linear_apply(g, P, 1, P, P, 2, P, P, None, None, P, lws, None) == _lib.VSA_ERR_LAYOUT
    assert lib.vsa_linear_apply(g, P, 2, P, P, 2, P, P, None, None, P, lws - 1, None) == _lib.VSA_ERR_WORKSPACE
    # Q / output layout: token-major or raster only.
    assert lib.vsa_linear_branch(g, P, 1, P, P, P, 2, P, P, None, None, P, lws, None) == _lib.VSA_ERR_LAYOUT
    assert lib.vsa_linear_branch(g, P, 7, P, P, P, 2, P, P, None, None, P, lws, None) == _lib.VSA_ERR_LAYOUT


def test_fused_entry_points_reject_bad_arguments(lib):
    from block_sparse_video_cube_amd import _lib

    g = geom()
    P = FAKE
    assert lib.vsa_cube_permute_pool(g, P, P, None, None) == _lib.VSA_ERR_NULL
    assert lib.vsa_cube_permute_pool(g, P, P, ODD, None) == _lib.VSA_ERR_ALIGN
    assert lib.vsa_cube_permute_pool(geom(D=16), P, P, P, None) == _lib.VSA_ERR_HEAD_DIM
    ws = lib.vsa_select_workspace_bytes(g)
    assert lib.vsa_select_topk_pooled(g, P, None, 2, P, P, ws, None) == _lib.VSA_ERR_NULL
    assert lib.vsa_select_topk_pooled(g, P, P, 0, P, P, ws, None) == _lib.VSA_ERR_TOPK
    assert lib.vsa_select_topk_pooled(g, P, P, 2, P, P, 16, None) == _lib.VSA_ERR_WORKSPACE


def test_sta_entry_points(lib):
    from block_sparse_video_cube_amd import _lib

    P = FAKE
    # list length: min(window, cubes) per axis; 0 for invalid windows or geometry
    assert lib.vsa_sta_topk(geom(grid=(16, 28, 52)), 3, 3, 3) == 27
    assert lib.vsa_sta_topk(geom(grid=(16, 28, 52)), 9, 1, 2) == 4 * 1 * 2
    assert lib.vsa_sta_topk(geom(grid=(21, 45, 80)), 3, 5, 7) == 3 * 5 * 7
    assert lib.vsa_sta_topk(geom(grid=(5, 6, 7)), 3, 3, 3) == 8
    assert lib.vsa_sta_topk(geom(grid=(16, 28, 52)), 0, 3, 3) == 0
    assert lib.vsa_sta_topk(geom(B=0), 3, 3, 3) == 0
    g = geom()
    assert lib.vsa_sta_index(g, 3, 3, 3, None, None) == _lib.VSA_ERR_NULL
    assert lib.vsa_sta_index(g, 3, 3, 3, ODD, None) == _lib.VSA_ERR_ALIGN
    assert lib.vsa_sta_index(g, 3, 0, 3, P, None) == _lib.VSA_ERR_WINDOW
    assert lib.vsa_sta_index(g, 3, 3, -1, P, None) == _lib.VSA_ERR_WINDOW
    assert lib.vsa_sta_index(geom(D=48), 3, 3, 3, P, None) == _lib.VSA_ERR_HEAD_DIM


def test_backward_entry_point_validation(lib):
    from block_sparse_video_cube_amd import _lib

    g = geom()
    P = FAKE
    ws = lib.vsa_attn_bwd_workspace_bytes(g, 2)
    # delta and lse log2 e (B H Np f32 each) + counts + offsets (B H Nc) + lists (B H Nc k), each
    # 256-byte aligned
    assert ws >= 2 * 2 * 512 * 4 + 2 * 2 * 8 * 4 + 2 * 8 * 2 * 4
    assert lib.vsa_attn_bwd_workspace_bytes(g, 0) == 0
    assert lib.vsa_attn_bwd_workspace_bytes(g, 9) == 0
    args = [P] * 7  # qc kc vc oc doc lse idx
    outs = [P] * 3
    assert lib.vsa_sparse_attn_bwd(g, *args[:6], None, 2, 0.125, *outs, P, ws, None) == _lib.VSA_ERR_NULL
    assert lib.vsa_sparse_attn_bwd(g, *args, 2, 0.125, P, P, None, P, ws, None) == _lib.VSA_ERR_NULL
    assert lib.vsa_sparse_attn_bwd(g, ODD, *args[1:], 2, 0.125, *outs, P, ws, None) == _lib.VSA_ERR_ALIGN
    assert lib.vsa_sparse_attn_bwd(g, *args, 0, 0.125, *outs, P, ws, None) == _lib.VSA_ERR_TOPK
    assert lib.vsa_sparse_attn_bwd(g, *args, 9, 0.125, *outs, P, ws, None) == _lib.VSA_ERR_TOPK
    assert lib.vsa_sparse_attn_bwd(g, *args, 2, -1.0, *outs, P, ws, None) == _lib.VSA_ERR_SCALE
    assert lib.vsa_sparse_attn_bwd(g, *args, 2, float("nan"), *outs, P, ws, None) == _lib.VSA_ERR_SCALE
    assert lib.vsa_sparse_attn_bwd(g, *args, 2, 0.125, *outs, P, ws - 1, None) == _lib.VSA_ERR_WORKSPACE
    big = geom(grid=(4 * 17, 4 * 16, 4 * 16))
    assert lib.vsa_sparse_attn_bwd(big, *args, 2, 0.125, *outs, P, 1 << 40, None) == _lib.VSA_ERR_GEOMETRY


def test_raster_entry_point_validation(lib):
    from block_sparse_video_cube_amd import _lib

    g = geom()
    P = FAKE
    assert lib.vsa_cube_pool(g, P, None, None) == _lib.VSA_ERR_NULL
    assert lib.vsa_cube_pool(g, ODD, P, None) == _lib.VSA_ERR_ALIGN
    assert lib.vsa_cube_pool(geom(D=16), P, P, None) == _lib.VSA_ERR_HEAD_DIM
    R = _lib.VSA_LAYOUT_RASTER
    assert lib.vsa_sparse_attn_fwd_raster(g, P, P, R, P, P, 2, 0.125, None, None, None, None) == _lib.VSA_ERR_NULL
    assert lib.vsa_sparse_attn_fwd_raster(g, P, P, R, P, P, 2, 0.125, None, ODD, None, None) == _lib.VSA_ERR_ALIGN
    assert lib.vsa_sparse_attn_fwd_raster(g, P, ODD, R, P, P, 2, 0.125, P, None, None, None) == _lib.VSA_ERR_ALIGN
    assert lib.vsa_sparse_attn_fwd_raster(g, P, P, 1, P, P, 2, 0.125, P, None, None, None) == _lib.VSA_ERR_LAYOUT
    assert lib.vsa_sparse_attn_fwd_raster(g, P, P, R, P, P, 0, 0.125, P, None, None, None) == _lib.VSA_ERR_TOPK
    assert lib.vsa_sparse_attn_fwd_raster(g, P, P, 0, P, P, 2, 0.0, P, None, None, None) == _lib.VSA_ERR_SCALE
    # 32-bit buffer offsets: S * heads * D * 2 must stay below 2^31
    huge = geom(B=1, H=512, D=128, grid=(64, 64, 64))
    assert lib.vsa_sparse_attn_fwd_raster(huge, P, P, R, P, P, 2, 0.125, P, None, None, None) == _lib.VSA_ERR_GEOMETRY


def test_fp8_entry_point_validation(lib):
    from block_sparse_video_cube_amd import _lib

    g = geom()
    P = FAKE
    ws = lib.vsa_quant_fp8_workspace_bytes(g)
    assert ws == 512  # the head maxima of V, B x H x D fp32, rounded up to 256 bytes
    assert lib.vsa_quant_fp8_workspace_bytes(geom(D=16)) == 0
    qa = [P] * 10  # q k v q8 qscale k8 kscale v8t vscale qmean
    assert lib.vsa_quant_fp8(g, *qa[:9], None, None, None, ws, None) == _lib.VSA_ERR_NULL   # workspace
    assert lib.vsa_quant_fp8(g, None, *qa[1:], None, P, ws, None) == _lib.VSA_ERR_NULL
    assert lib.vsa_quant_fp8(g, *qa[:8], None, None, None, P, ws, None) == _lib.VSA_ERR_NULL  # vscale
    assert lib.vsa_quant_fp8(g, *qa[:3], ODD, *qa[4:], None, P, ws, None) == _lib.VSA_ERR_ALIGN
    assert lib.vsa_quant_fp8(g, *qa, ODD, P, ws, None) == _lib.VSA_ERR_ALIGN               # kmean
    assert lib.vsa_quant_fp8(g, *qa, None, P, ws - 1, None) == _lib.VSA_ERR_WORKSPACE
    assert lib.vsa_quant_fp8(geom(D=16), *qa, None, P, ws, None) == _lib.VSA_ERR_HEAD_DIM
    args = [P] * 7  # q8 qscale k8 kscale v8t vscale idx
    f = lib.vsa_sparse_attn_fwd_fp8
    TM = _lib.VSA_LAYOUT_TOKEN_MAJOR
    assert f(g, *args, 2, 0.125, TM, None, None, None) == _lib.VSA_ERR_NULL
    assert f(g, *args[:6], None, 2, 0.125, TM, P, None, None) == _lib.VSA_ERR_NULL
    assert f(g, ODD, *args[1:], 2, 0.125, TM, P, None, None) == _lib.VSA_ERR_ALIGN
    assert f(g, *args, 2, 0.125, TM, P, ODD, None) == _lib.VSA_ERR_ALIGN
    assert f(g, *args, 0, 0.125, TM, P, None, None) == _lib.VSA_ERR_TOPK
    assert f(g, *args, 9, 0.125, TM, P, None, None) == _lib.VSA_ERR_TOPK
    assert f(g, *args, 2, float("inf"), TM, P, None, None) == _lib.VSA_ERR_SCALE
    assert f(g, *args, 2, 0.125, _lib.VSA_LAYOUT_DIM_MAJOR, P, None, None) == _lib.VSA_ERR_LAYOUT
    assert f(geom(D=96), *args, 2, 0.125, TM, P, None, None) == _lib.VSA_ERR_HEAD_DIM

def test_fused_linear_entry_point_validation(lib):
    from block_sparse_video_cube_amd import _lib

    g = geom()
    P = FAKE
    ws = lib.vsa_linear_workspace_bytes(g)
    f = lib.vsa_sparse_attn_linear_fwd
    assert f(g, P, P, P, P, 2, 0.125, None, None, P, ws, None) == _lib.VSA_ERR_NULL
    assert f(g, P, P, P, P, 2, 0.125, P, None, None, ws, None) == _lib.VSA_ERR_NULL
    assert f(g, P, ODD, P, P, 2, 0.125, P, None, P, ws, None) == _lib.VSA_ERR_ALIGN
    assert f(g, P, P, P, P, 2, 0.125, P, ODD, P, ws, None) == _lib.VSA_ERR_ALIGN
    assert f(g, P, P, P, P, 0, 0.125, P, None, P, ws, None) == _lib.VSA_ERR_TOPK
    assert f(g, P, P, P, P, 9, 0.125, P, None, P, ws, None) == _lib.VSA_ERR_TOPK
    assert f(g, P, P, P, P, 5, 0.125, P, None, P, ws, None) == _lib.VSA_ERR_TOPK  # more than half, not all
    assert f(g, P, P, P, P, 2, float("nan"), P, None, P, ws, None) == _lib.VSA_ERR_SCALE
    assert f(g, P, P, P, P, 2, 0.125, P, None, P, ws - 1, None) == _lib.VSA_ERR_WORKSPACE
    assert f(geom(D=32), P, P, P, P, 2, 0.125, P, None, P, ws, None) == _lib.VSA_ERR_HEAD_DIM


def test_mfma_probe_validation(lib):
    from block_sparse_video_cube_amd import _lib

    P = FAKE
    assert lib.vsa_mfma_probe(8, 10, None, P, None) == _lib.VSA_ERR_NULL
    assert lib.vsa_mfma_probe(8, 10, P, None, None) == _lib.VSA_ERR_NULL
    assert lib.vsa_mfma_probe(8, 10, ODD, P, None) == _lib.VSA_ERR_ALIGN
    assert lib.vsa_mfma_probe(0, 10, P, P, None) == _lib.VSA_ERR_GEOMETRY
    assert lib.vsa_mfma_probe(8, 0, P, P, None) == _lib.VSA_ERR_GEOMETRY
    assert lib.vsa_mfma_probe((1 << 20) + 1, 10, P, P, None) == _lib.VSA_ERR_GEOMETRY


def test_hbm_probe_validation(lib):
    from block_sparse_video_cube_amd import _lib

    P = FAKE
    assert lib.vsa_hbm_probe(3, P, P, 1024, None) == _lib.VSA_ERR_LAYOUT
    assert lib.vsa_hbm_probe(-1, P, P, 1024, None) == _lib.VSA_ERR_LAYOUT
    assert lib.vsa_hbm_probe(0, None, P, 1024, None) == _lib.VSA_ERR_NULL
    assert lib.vsa_hbm_probe(0, P, None, 1024, None) == _lib.VSA_ERR_NULL
    assert lib.vsa_hbm_probe(1, None, None, 1024, None) == _lib.VSA_ERR_NULL
    assert lib.vsa_hbm_probe(2, None, None, 1024, None) == _lib.VSA_ERR_NULL
    assert lib.vsa_hbm_probe(0, ODD, P, 1024, None) == _lib.VSA_ERR_ALIGN
    assert lib.vsa_hbm_probe(0, P, P, 1000, None) == _lib.VSA_ERR_GEOMETRY
    assert lib.vsa_hbm_probe(2, None, P, 0, None) == _lib.VSA_ERR_GEOMETRY
    assert lib.vsa_hbm_probe(1, P, None, (1 << 40) + 16, None) == _lib.VSA_ERR_GEOMETRY


def test_linear_backward_entry_point_validation(lib):
    from block_sparse_video_cube_amd import _lib

    g = geom()
    P = FAKE
    ws = lib.vsa_linear_bwd_workspace_bytes(g, 2)
    assert ws >= lib.vsa_linear_workspace_bytes(g)
    assert lib.vsa_linear_bwd_workspace_bytes(g, 0) == 0
    assert lib.vsa_linear_bwd_workspace_bytes(g, 9) == 0
    ins = [P] * 5  # qc kc vc vt idx
    saved = [None] * 2  # o_lin, inv_den
    adds = [None] * 3
    outs = [P] * 3
    assert lib.vsa_linear_branch_bwd(g, *ins, 2, None, *saved, *adds, *outs, P, ws, None) == _lib.VSA_ERR_NULL
    assert lib.vsa_linear_branch_bwd(g, *ins, 2, P, *saved, *adds, P, P, None, P, ws, None) == _lib.VSA_ERR_NULL
    assert lib.vsa_linear_branch_bwd(g, ODD, *ins[1:], 2, P, *saved, *adds, *outs, P, ws, None) == _lib.VSA_ERR_ALIGN
    assert lib.vsa_linear_branch_bwd(g, *ins, 2, P, *saved, ODD, None, None, *outs, P, ws, None) == _lib.VSA_ERR_ALIGN
    assert lib.vsa_linear_branch_bwd(g, *ins, 0, P, *saved, *adds, *outs, P, ws, None) == _lib.VSA_ERR_TOPK
    assert lib.vsa_linear_branch_bwd(g, *ins, 9, P, *saved, *adds, *outs, P, ws, None) == _lib.VSA_ERR_TOPK
    assert lib.vsa_linear_branch_bwd(g, *ins, 2, P, *saved, *adds, *outs, P, ws - 1, None) == _lib.VSA_ERR_WORKSPACE
    assert lib.vsa_linear_branch_bwd(geom(D=48), *ins, 2, P, *saved, *adds, *outs, P, ws, None) == \
        _lib.VSA_ERR_HEAD_DIM
    # The saved forward values: a pair, 16-byte aligned.
    assert lib.vsa_linear_branch_bwd(g, *ins, 2, P, P, None, *adds, *outs, P, ws, None) == _lib.VSA_ERR_NULL
    assert lib.vsa_linear_branch_bwd(g, *ins, 2, P, None, P, *adds, *outs, P, ws, None) == _lib.VSA_ERR_NULL
    assert lib.vsa_linear_branch_bwd(g, *ins, 2, P, P, ODD, *adds, *outs, P, ws, None) == _lib.VSA_ERR_ALIGN


def test_packed_entry_point_validation(lib):
    from block_sparse_video_cube_amd import _lib

    P = FAKE
    R, T = _lib.VSA_LAYOUT_RASTER, _lib.VSA_LAYOUT_TOKEN_MAJOR
    full = geom(grid=(8, 8, 8))
    part = geom(grid=(5, 6, 7))
    # Workspace: the packing plan (16 bytes per tile and per row header), then
    # the launch order (an int32 per query cube, rounded up to 256 bytes);
    # none for full grids.
    assert lib.vsa_sparse_attn_packed_workspace_bytes(full, 2) == 0
    assert lib.vsa_sparse_attn_packed_workspace_bytes(part, 3) == 1 * 2 * 8 * 16 * 4 + 256
    assert lib.vsa_sparse_attn_packed_workspace_bytes(part, 0) == 0
    assert lib.vsa_sparse_attn_packed_workspace_bytes(part, 9) == 0
    ws = lib.vsa_sparse_attn_packed_workspace_bytes(part, 3)
    f = lib.vsa_sparse_attn_fwd_packed
    assert f(part, P, R, P, P, P, 3, 0.125, P, None, None, ws, None) == _lib.VSA_ERR_NULL
    assert f(part, P, R, P, P, P, 3, 0.125, P, None, P, ws - 1, None) == _lib.VSA_ERR_WORKSPACE
    assert f(part, P, R, P, P, P, 3, 0.125, P, None, ODD, ws, None) == _lib.VSA_ERR_ALIGN
    assert f(part, P, 1, P, P, P, 3, 0.125, P, None, P, ws, None) == _lib.VSA_ERR_LAYOUT
    assert f(part, P, R, P, P, P, 0, 0.125, P, None, P, ws, None) == _lib.VSA_ERR_TOPK
    assert f(part, P, T, P, P, P, 3, -1.0, P, None, P, ws, None) == _lib.VSA_ERR_SCALE
    assert f(part, P, R, None, P, P, 3, 0.125, P, None, P, ws, None) == _lib.VSA_ERR_NULL
    assert f(part, P, R, P, P, P, 3, 0.125, P, ODD, P, ws, None) == _lib.VSA_ERR_ALIGN
    # A full grid needs no workspace, but the other checks still apply.
    assert f(full, P, R, P, P, P, 9, 0.125, P, None, None, 0, None) == _lib.VSA_ERR_TOPK
    assert f(geom(D=32), P, R, P, P, P, 2, 0.125, P, None, None, 0, None) == _lib.VSA_ERR_HEAD_DIM
    # Compact permutes.
    assert lib.vsa_cube_permute(part, P, None, _lib.VSA_LAYOUT_TOKEN_COMPACT, None) == _lib.VSA_ERR_NULL
    assert lib.vsa_cube_permute(part, None, P, _lib.VSA_LAYOUT_DIM_SLOTS, None) == _lib.VSA_ERR_NULL
    assert lib.vsa_cube_permute(part, P, P, 5, None) == _lib.VSA_ERR_LAYOUT
    assert lib.vsa_cube_permute_pool_compact(part, P, None, P, None) == _lib.VSA_ERR_NULL
    assert lib.vsa_cube_permute_pool_compact(part, P, P, ODD, None) == _lib.VSA_ERR_ALIGN


def test_geom_dims_reject_axes_that_overflow(lib):
    # Axes near INT32_MAX: the cube counts are checked before any narrowing
    # or product can overflow.
    from block_sparse_video_cube_amd import _lib

    d = _lib.VsaDims()
    for grid in [(2**31 - 1, 2**31 - 1, 1), (2**31 - 1, 1, 1), (1, 2**26 + 1, 1), (2**13, 2**13, 2**13)]:
        assert lib.vsa_geom_dims(geom(grid=grid), ctypes.byref(d)) == _lib.VSA_ERR_GEOMETRY, grid
    assert lib.vsa_geom_dims(geom(B=1, H=1, grid=(2**26, 1, 1)), ctypes.byref(d)) == 0
    assert d.n_cubes == 2**24 and d.pad_t == 2**26
