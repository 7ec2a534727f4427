"""The Python binding on a host without a GPU: it marshals arguments only.

Every public operation refuses tensors that are not on the GPU (there is no
CPU fallback), checks shapes before anything is launched, and the package
imports nothing from the oracle.
"""

import subprocess
import sys

import pytest
import torch

import workloads

GRID = (8, 8, 8)


def bf16(*shape):
    return torch.zeros(shape, dtype=torch.bfloat16)


@pytest.fixture(scope="module")
def vsa():
    import block_sparse_video_cube_amd as m

    return m


def calls(vsa):
    B, S, H, D = 1, 512, 2, 64
    x = bf16(B, S, H, D)
    qc = bf16(B, H, 512, D)
    vt = bf16(B, H, 8, D, 64)
    idx = torch.zeros((B, H, 8, 2), dtype=torch.int32)
    means = torch.zeros((B, H, 8, D), dtype=torch.float32)
    u8 = torch.zeros((B, H, 512, D), dtype=torch.uint8)
    sc = torch.zeros((B, H, 8), dtype=torch.float32)
    v8t = torch.zeros((B, H, 8, D, 64), dtype=torch.uint8)
    vs = torch.zeros((B, H, D), dtype=torch.float32)
    lse = torch.zeros((B, H, 512), dtype=torch.float32)
    return {
        "cube_permute": lambda: vsa.cube_permute(x, GRID),
        "cube_permute_pool": lambda: vsa.cube_permute_pool(x, GRID),
        "cube_pool": lambda: vsa.cube_pool(x, GRID),
        "cube_unpermute": lambda: vsa.cube_unpermute(qc, GRID),
        "select_topk": lambda: vsa.select_topk(qc, qc, GRID, 2),
        "select_topk_pooled": lambda: vsa.select_topk_pooled(means, means, GRID, 2),
        "sparse_attn_fwd": lambda: vsa.sparse_attn_fwd(qc, qc, vt, idx, GRID),
        "sparse_attn_fwd_raster": lambda: vsa.sparse_attn_fwd_raster(x, qc, vt, idx, GRID),
        "sparse_attn_linear_fwd": lambda: vsa.sparse_attn_linear_fwd(qc, qc, vt, idx, GRID),
        "quant_fp8": lambda: vsa.quant_fp8(x, x, x, GRID),
        "sparse_attn_fwd_fp8": lambda: vsa.sparse_attn_fwd_fp8(u8, sc, u8, sc, v8t, vs, idx, GRID),
        "sparse_attn_bwd": lambda: vsa.sparse_attn_bwd(qc, qc, qc, qc, qc, lse, idx, GRID),
        "linear_branch_bwd": lambda: vsa.linear_branch_bwd(qc, qc, qc, vt, idx, qc, GRID),
    }


NAMES = ["cube_permute", "cube_permute_pool", "cube_pool", "cube_unpermute", "select_topk", "select_topk_pooled",
         "sparse_attn_fwd", "sparse_attn_fwd_raster", "sparse_attn_linear_fwd", "quant_fp8", "sparse_attn_fwd_fp8",
         "sparse_attn_bwd", "linear_branch_bwd"]


@pytest.mark.parametrize("name", NAMES)
def test_host_tensors_are_refused(vsa, name):
    with pytest.raises(ValueError, match="on the GPU"):
        calls(vsa)[name]()


def test_argument_checks(vsa):
    from block_sparse_video_cube_amd import _need

    t = torch.zeros((2, 3), dtype=torch.float32)
    with pytest.raises(TypeError):
        _need([0.0], "x", torch.float32, (2, 3))
    with pytest.raises(ValueError, match="on the GPU"):
        _need(t, "x", torch.float32, (2, 3))


def test_package_does_not_import_the_oracle():
    code = ("import sys; import block_sparse_video_cube_amd as m; import block_sparse_video_cube_amd.build; "
            "print(int(any(k == 'oracle' or k.startswith('oracle.') for k in sys.modules)))")
    out = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, cwd=workloads.__file__.rsplit(
        "/workloads", 1)[0])
    assert out.returncode == 0, out.stderr
    assert out.stdout.strip() == "0"
