"""GPU parity of the raster-order (gather-on-load) fine stage and of pooling
without the cube-major copy.

Both compute exactly what the cube-major path computes, in the same order,
so they are compared bit for bit with it (vsa_cube_permute_pool means;
vsa_sparse_attn_fwd followed by vsa_cube_unpermute, and its lse), and once
against the oracle within the bf16 output tolerance.
"""

import numpy as np
import pytest
import torch

import oracle
import workloads
from tests.gpu_util import assert_close, to_bits, to_dev

pytestmark = pytest.mark.gpu

CASES = [
    # (B, H, D, grid, k)
    (1, 2, 64, (8, 8, 8), 2),
    (2, 3, 128, (8, 12, 16), 5),
    (1, 2, 128, (9, 14, 13), 4),    # partial cubes on every axis
    (1, 1, 64, (5, 6, 7), 3),
    (1, 2, 128, (21, 9, 16), 7),    # partial along t only
]


def run_both(B, H, D, grid, k, seed=3000):
    import block_sparse_video_cube_amd as vsa

    wl = workloads.workload("tiny").with_(batch=B, heads=H, head_dim=D, grid=grid, topk=k, seed=seed)
    inp = workloads.make_inputs(wl)
    q, kk, v = (to_dev(inp[n]) for n in ("q", "k", "v"))
    qc, qbar = vsa.cube_permute_pool(q, grid)
    kc, kbar = vsa.cube_permute_pool(kk, grid)
    vt = vsa.cube_permute(v, grid, layout="dim")
    idx = vsa.select_topk_pooled(qbar, kbar, grid, k)
    oc, _, lse_c = vsa.sparse_attn_fwd(qc, kc, vt, idx, grid, wl.softmax_scale, want_lse=True)
    o_ref = vsa.cube_unpermute(oc, grid)
    o_r, lse_r = vsa.sparse_attn_fwd_raster(q, kk, vt, idx, grid, wl.softmax_scale, want_lse=True)  # K gathered
    o_k, lse_k = vsa.sparse_attn_fwd_raster(q, kc, vt, idx, grid, wl.softmax_scale, want_lse=True)  # K cube-major
    qbar2 = vsa.cube_pool(q, grid)
    kbar2 = vsa.cube_pool(kk, grid)
    torch.cuda.synchronize()
    return wl, inp, idx, (qbar, kbar, qbar2, kbar2), (o_ref, o_r, o_k), (lse_c, lse_r, lse_k)


@pytest.mark.parametrize("B,H,D,grid,k", CASES)
def test_raster_path_bit_identical_to_cube_major(B, H, D, grid, k):
    wl, inp, idx, means, outs, lses = run_both(B, H, D, grid, k)
    qbar, kbar, qbar2, kbar2 = means
    assert torch.equal(qbar, qbar2) and torch.equal(kbar, kbar2)
    assert torch.equal(outs[0], outs[1]) and torch.equal(outs[0], outs[2])
    valid = torch.from_numpy(oracle.valid_rows(grid)).to(lses[0].device)
    assert torch.equal(lses[0][:, :, valid], lses[1][:, :, valid])
    assert torch.equal(lses[0][:, :, valid], lses[2][:, :, valid])


def test_raster_path_matches_oracle():
    B, H, D, grid, k = 1, 2, 128, (9, 14, 13), 4
    wl, inp, idx, _, outs, _ = run_both(B, H, D, grid, k, seed=3100)
    ref, _ = oracle.forward(inp["q"], inp["k"], inp["v"], grid, k, idx=idx.cpu().numpy())
    assert_close(oracle.bf16_to_f64(to_bits(outs[1])), ref, "raster fine stage vs oracle")


@pytest.mark.parametrize("name", ["wan1.3b", "720p"])
def test_raster_path_full_size_bit_identical(name):
    import block_sparse_video_cube_amd as vsa

    wl = workloads.workload(name)
    inp = workloads.make_inputs(wl)
    q, kk, v = (to_dev(inp[n]) for n in ("q", "k", "v"))
    del inp
    kbar = vsa.cube_pool(kk, wl.grid)
    qbar = vsa.cube_pool(q, wl.grid)
    vt = vsa.cube_permute(v, wl.grid, layout="dim")
    idx = vsa.select_topk_pooled(qbar, kbar, wl.grid, wl.topk)
    o_r, _ = vsa.sparse_attn_fwd_raster(q, kk, vt, idx, wl.grid, wl.softmax_scale)
    qc = vsa.cube_permute(q, wl.grid)
    kc = vsa.cube_permute(kk, wl.grid)
    oc, _, _ = vsa.sparse_attn_fwd(qc, kc, vt, idx, wl.grid, wl.softmax_scale)
    o_c = vsa.cube_unpermute(oc, wl.grid)
    o_k, _ = vsa.sparse_attn_fwd_raster(q, kc, vt, idx, wl.grid, wl.softmax_scale)
    torch.cuda.synchronize()
    assert torch.isfinite(o_r.float()).all()
    assert torch.equal(o_r, o_c) and torch.equal(o_k, o_c)
