"""ctypes declarations of the C ABI in include/vsa_cube.h."""

from __future__ import annotations

import ctypes
import os

LIB_NAME = "libvsa_cube.so"
LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), LIB_NAME)

VSA_OK = 0
VSA_ERR_NULL = 1
VSA_ERR_GEOMETRY = 2
VSA_ERR_HEAD_DIM = 3
VSA_ERR_TOPK = 4
VSA_ERR_ALIGN = 5
VSA_ERR_WORKSPACE = 6
VSA_ERR_LAYOUT = 7
VSA_ERR_SCALE = 8
VSA_ERR_LAUNCH = 9
VSA_ERR_WINDOW = 10
VSA_ERR_SCRATCH = 11
VSA_QUANT_SCRATCH_WORDS = 65536

VSA_LAYOUT_TOKEN_MAJOR = 0
VSA_LAYOUT_DIM_MAJOR = 1
VSA_LAYOUT_RASTER = 2
VSA_LAYOUT_TOKEN_COMPACT = 3
VSA_LAYOUT_DIM_SLOTS = 4
VSA_MAX_CUBES = 4096

ENTRY_POINTS = (
    "vsa_abi_version",
    "vsa_status_string",
    "vsa_geom_dims",
    "vsa_select_workspace_bytes",
    "vsa_linear_workspace_bytes",
    "vsa_cube_permute",
    "vsa_cube_permute_pool",
    "vsa_cube_unpermute",
    "vsa_select_topk",
    "vsa_select_topk_pooled",
    "vsa_sparse_attn_fwd",
    "vsa_linear_branch",
    "vsa_linear_state",
    "vsa_linear_apply",
    "vsa_linear_states_bytes",
    "vsa_linear_unselected_bytes",
    "vsa_linear_unselected_workspace_bytes",
    "vsa_linear_cube_states",
    "vsa_linear_unselected",
    "vsa_sparse_attn_fwd_linear",
    "vsa_sta_topk",
    "vsa_sta_index",
    "vsa_cube_pool",
    "vsa_sparse_attn_fwd_raster",
    "vsa_attn_bwd_workspace_bytes",
    "vsa_sparse_attn_bwd",
    "vsa_quant_fp8_workspace_bytes",
    "vsa_quant_fp8",
    "vsa_quant_fp8_packed",
    "vsa_sparse_attn_fwd_fp8",
    "vsa_sparse_attn_fwd_fp8_packed",
    "vsa_sparse_attn_linear_fwd",
    "vsa_mfma_probe",
    "vsa_hbm_probe",
    "vsa_linear_bwd_workspace_bytes",
    "vsa_linear_branch_bwd",
    "vsa_cube_permute_pool_compact",
    "vsa_sparse_attn_packed_workspace_bytes",
    "vsa_sparse_attn_fwd_packed",
    "vsa_quant_fp8_noalloc",
)


class VsaGeom(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("grid_t", ctypes.c_int32),
        ("grid_h", ctypes.c_int32),
        ("grid_w", ctypes.c_int32),
    ]


class VsaDims(ctypes.Structure):
    _fields_ = [
        ("pad_t", ctypes.c_int32),
        ("pad_h", ctypes.c_int32),
        ("pad_w", ctypes.c_int32),
        ("cubes_t", ctypes.c_int32),
        ("cubes_h", ctypes.c_int32),
        ("cubes_w", ctypes.c_int32),
        ("n_cubes", ctypes.c_int32),
        ("reserved", ctypes.c_int32),
        ("tokens", ctypes.c_int64),
        ("rows", ctypes.c_int64),
    ]


_lib = None


class VsaError(RuntimeError):
    def __init__(self, fn: str, status: int, text: str):
        super().__init__(f"{fn} failed with status {status}: {text}")
        self.status = status


def load() -> ctypes.CDLL:
    """Load the built library; raise if it is missing (there is no fallback)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is missing: build the HIP library first "
            "(python -c 'import __graft_entry__ as g; g.build()')")
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.c_void_p
    G = ctypes.POINTER(VsaGeom)
    i32 = ctypes.c_int32
    sz = ctypes.c_size_t
    sig = {
        "vsa_abi_version": (i32, []),
        "vsa_status_string": (ctypes.c_char_p, [i32]),
        "vsa_geom_dims": (i32, [G, ctypes.POINTER(VsaDims)]),
        "vsa_select_workspace_bytes": (sz, [G]),
        "vsa_linear_workspace_bytes": (sz, [G]),
        "vsa_cube_permute": (i32, [G, P, P, i32, P]),
        "vsa_cube_permute_pool": (i32, [G, P, P, P, P]),
        "vsa_select_topk_pooled": (i32, [G, P, P, i32, P, P, sz, P]),
        "vsa_cube_unpermute": (i32, [G, P, P, P]),
        "vsa_select_topk": (i32, [G, P, P, i32, P, P, sz, P]),
        "vsa_sparse_attn_fwd": (i32, [G, P, P, P, P, i32, ctypes.c_float, P, P, P, P]),
        "vsa_linear_branch": (i32, [G, P, i32, P, P, P, i32, P, P, P, P, P, sz, P]),
        "vsa_linear_state": (i32, [G, P, P, P, sz, P]),
        "vsa_linear_apply": (i32, [G, P, i32, P, P, i32, P, P, P, P, P, sz, P]),
        "vsa_linear_states_bytes": (sz, [G]),
        "vsa_linear_unselected_bytes": (sz, [G]),
        "vsa_linear_unselected_workspace_bytes": (sz, [G]),
        "vsa_linear_cube_states": (i32, [G, P, P, P, P]),
        "vsa_linear_unselected": (i32, [G, P, P, i32, P, P, sz, P]),
        "vsa_sparse_attn_fwd_linear": (i32, [G, P, i32, P, P, P, i32, ctypes.c_float, P, P, P, P]),
        "vsa_sta_topk": (i32, [G, i32, i32, i32]),
        "vsa_sta_index": (i32, [G, i32, i32, i32, P, P]),
        "vsa_cube_pool": (i32, [G, P, P, P]),
        "vsa_sparse_attn_fwd_raster": (i32, [G, P, P, i32, P, P, i32, ctypes.c_float, P, P, P, P]),
        "vsa_attn_bwd_workspace_bytes": (sz, [G, i32]),
        "vsa_quant_fp8_workspace_bytes": (sz, [G]),
        "vsa_quant_fp8": (i32, [G, P, P, P, P, P, P, P, P, P, P, P, P, sz, P]),
        "vsa_sparse_attn_fwd_fp8": (i32, [G, P, P, P, P, P, P, P, i32, ctypes.c_float, i32, P, P, P]),
        "vsa_quant_fp8_packed": (i32, [G, P, P, P, P, P, P, P, P, P, P, P, P, sz, P]),
        "vsa_sparse_attn_fwd_fp8_packed": (i32, [G, P, P, P, P, P, P, P, i32, ctypes.c_float, i32, P, P, P, sz, P]),
        "vsa_sparse_attn_linear_fwd": (i32, [G, P, P, P, P, i32, ctypes.c_float, P, P, P, sz, P]),
        "vsa_sparse_attn_bwd": (i32, [G, P, P, P, P, P, P, P, i32, ctypes.c_float, P, P, P, P, sz, P]),
        "vsa_mfma_probe": (i32, [i32, i32, P, P, P]),
        "vsa_hbm_probe": (i32, [i32, P, P, sz, P]),
        "vsa_linear_bwd_workspace_bytes": (sz, [G, i32]),
        "vsa_linear_branch_bwd": (i32, [G, P, P, P, P, P, i32, P, P, P, P, P, P, P, P, P, P, sz, P]),
        "vsa_cube_permute_pool_compact": (i32, [G, P, P, P, P]),
        "vsa_sparse_attn_packed_workspace_bytes": (sz, [G, i32]),
        "vsa_sparse_attn_fwd_packed": (i32, [G, P, i32, P, P, P, i32, ctypes.c_float, P, P, P, sz, P]),
        "vsa_quant_fp8_noalloc": (i32, [G, P, P, P, P, P, P, P, P, P, P, P, P]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def check(fn: str, status: int) -> None:
    if status != VSA_OK:
        text = load().vsa_status_string(status).decode()
        raise VsaError(fn, status, text)
