"""GPU parity of the sliding-tile (STA) pattern.

Block lists: bit-exact against the oracle's sliding-tile lists (integer work).
Fine stage fed those lists: within the bf16 output tolerance of the oracle's
sparse attention over the same lists, at small sizes in full and at the
Wan2.1-1.3B workload size on sampled query cubes.
"""

import numpy as np
import pytest
import torch

import oracle
import workloads
from tests.gpu_util import assert_close, to_bits, to_dev

pytestmark = pytest.mark.gpu

INDEX_CASES = [
    # (B, H, grid, window)
    (1, 1, (8, 8, 8), (3, 3, 3)),
    (2, 3, (16, 28, 52), (3, 3, 3)),
    (1, 2, (21, 45, 80), (3, 5, 7)),
    (1, 1, (5, 6, 7), (2, 4, 3)),
    (1, 1, (12, 4, 20), (9, 9, 9)),   # wider than the grid on every axis: dense
    (1, 2, (16, 28, 52), (1, 1, 1)),  # own cube only
    (1, 1, (4, 4, 4), (1, 2, 1)),     # a single cube
]


@pytest.mark.parametrize("B,H,grid,window", INDEX_CASES)
def test_sta_index_bit_exact(B, H, grid, window):
    import block_sparse_video_cube_amd as vsa

    ref = oracle.sta_index(grid, window)
    assert vsa.sta_topk(grid, window) == ref.shape[1]
    got = vsa.sta_index(grid, window, B, H).cpu().numpy()
    assert got.shape == (B, H) + ref.shape
    for b in range(B):
        for h in range(H):
            assert np.array_equal(got[b, h], ref)


@pytest.mark.parametrize("D,grid,window", [
    (64, (8, 12, 16), (3, 3, 3)),
    (128, (8, 12, 16), (2, 3, 3)),
    (128, (9, 14, 13), (3, 3, 3)),   # partial cubes on every axis
    (64, (5, 6, 7), (3, 3, 3)),      # window wider than the 2x2x2 cube grid
])
def test_sta_fine_stage_matches_oracle(D, grid, window):
    import block_sparse_video_cube_amd as vsa

    wl = workloads.workload("tiny").with_(batch=1, heads=2, head_dim=D, grid=grid)
    inp = workloads.make_inputs(wl)
    q, k, v = (to_dev(inp[n]) for n in ("q", "k", "v"))
    qc = vsa.cube_permute(q, grid)
    kc = vsa.cube_permute(k, grid)
    vt = vsa.cube_permute(v, grid, layout="dim")
    idx = vsa.sta_index(grid, window, 1, 2, head_dim=D)
    oc, _, _ = vsa.sparse_attn_fwd(qc, kc, vt, idx, grid, wl.softmax_scale)
    o = vsa.cube_unpermute(oc, grid)
    torch.cuda.synchronize()
    idx_o = np.broadcast_to(oracle.sta_index(grid, window), idx.shape)
    ref, _ = oracle.forward(inp["q"], inp["k"], inp["v"], grid, idx_o.shape[-1], idx=idx_o)
    assert_close(oracle.bf16_to_f64(to_bits(o)), ref, f"sta D={D} grid={grid} window={window}")


def test_sta_workload_sampled():
    import block_sparse_video_cube_amd as vsa

    wl = workloads.workload("sta")
    heads = [0, 7]
    inp = workloads.make_inputs(wl)
    q, k, v = (to_dev(inp[n]) for n in ("q", "k", "v"))
    qc = vsa.cube_permute(q, wl.grid)
    kc = vsa.cube_permute(k, wl.grid)
    vt = vsa.cube_permute(v, wl.grid, layout="dim")
    idx = vsa.sta_index(wl.grid, wl.window, wl.batch, wl.heads)
    assert idx.shape[-1] == wl.topk
    oc, _, _ = vsa.sparse_attn_fwd(qc, kc, vt, idx, wl.grid, wl.softmax_scale)
    torch.cuda.synchronize()
    ref_idx = oracle.sta_index(wl.grid, wl.window)
    assert np.array_equal(idx.cpu().numpy()[0, 3], ref_idx)
    rng = np.random.default_rng(7)
    cubes = sorted({0, wl.n_cubes - 1, *(int(c) for c in rng.choice(wl.n_cubes, 16, replace=False))})
    sub = {n: np.ascontiguousarray(inp[n][:, :, heads, :]) for n in ("q", "k", "v")}
    valid = oracle.valid_rows(wl.grid)
    qc_o, kc_o, vc_o = (oracle.cube_permute(sub[n], wl.grid) for n in ("q", "k", "v"))
    idx_o = np.broadcast_to(ref_idx, (1, len(heads)) + ref_idx.shape)
    want = [(0, hi, c) for hi in range(len(heads)) for c in cubes]
    ref, _ = oracle.sparse_attention(qc_o, kc_o, vc_o, valid, idx_o, wl.softmax_scale, cubes=want)
    got = oracle.bf16_to_f64(to_bits(oc[:, heads]))
    rows = np.concatenate([np.arange(64 * c, 64 * c + 64) for c in cubes])
    assert_close(got[:, :, rows], ref[:, :, rows], "sta workload sampled cubes")
