"""GPU parity: cube permutation and its inverse, bit-exact against the oracle."""

import numpy as np
import pytest
import torch

import oracle
import workloads
from tests.gpu_util import to_bits, to_dev

pytestmark = pytest.mark.gpu

CASES = [
    # (B, H, D, grid)
    (1, 2, 64, (8, 8, 8)),
    (2, 3, 128, (5, 6, 7)),
    (1, 1, 64, (1, 1, 1)),
    (1, 2, 128, (9, 3, 13)),
    (2, 1, 64, (4, 4, 4)),
    (1, 4, 128, (21, 9, 16)),
]


def rand_bits(shape, seed):
    rng = np.random.default_rng(seed)
    return rng.integers(0, 1 << 16, size=shape).astype(np.uint16) & np.uint16(0x7F7F) | np.uint16(0x0080)


@pytest.mark.parametrize("B,H,D,grid", CASES)
def test_permute_token_major_bit_exact(B, H, D, grid):
    import block_sparse_video_cube_amd as vsa

    S = grid[0] * grid[1] * grid[2]
    x = rand_bits((B, S, H, D), 1)
    got = to_bits(vsa.cube_permute(to_dev(x), grid))
    ref = oracle.cube_permute(x, grid)
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("B,H,D,grid", CASES)
def test_permute_dim_major_bit_exact(B, H, D, grid):
    import block_sparse_video_cube_amd as vsa

    S = grid[0] * grid[1] * grid[2]
    x = rand_bits((B, S, H, D), 2)
    got = to_bits(vsa.cube_permute(to_dev(x), grid, layout="dim"))
    ref = oracle.cube_permute(x, grid)  # [B, H, Np, D]
    nc = oracle.n_cubes(grid)
    ref_t = ref.reshape(B, H, nc, 64, D).transpose(0, 1, 2, 4, 3)
    assert np.array_equal(got, ref_t)


@pytest.mark.parametrize("B,H,D,grid", CASES)
def test_unpermute_bit_exact_and_drops_pads(B, H, D, grid):
    import block_sparse_video_cube_amd as vsa

    nc = oracle.n_cubes(grid)
    xc = rand_bits((B, H, nc * 64, D), 3)  # pads hold garbage on purpose
    got = to_bits(vsa.cube_unpermute(to_dev(xc), grid))
    assert np.array_equal(got, oracle.cube_unpermute(xc, grid))


def test_roundtrip_720p_shape_one_head():
    import block_sparse_video_cube_amd as vsa

    wl = workloads.workload("720p")
    x = workloads.make_head(wl, "q", 0, 5)[None, :, None, :]
    xd = to_dev(x)
    xc = vsa.cube_permute(xd, wl.grid)
    assert xc.shape == (1, 1, wl.rows, 128)
    back = vsa.cube_unpermute(xc, wl.grid)
    assert torch.equal(back, xd)
    # Sampled rows against the oracle's index map.
    xcb = to_bits(xc)[0, 0]
    rng = np.random.default_rng(4)
    T, H, W = wl.grid
    for _ in range(500):
        t, y, xx = int(rng.integers(T)), int(rng.integers(H)), int(rng.integers(W))
        c, l = oracle.token_row(t, y, xx, wl.grid)
        assert np.array_equal(xcb[64 * c + l], x[0, (t * H + y) * W + xx, 0])
    valid = oracle.valid_rows(wl.grid)
    assert np.all(xcb[~valid] == 0)


@pytest.mark.parametrize("B,H,D,grid", CASES)
def test_permute_pool_rows_and_means(B, H, D, grid):
    import block_sparse_video_cube_amd as vsa

    wl = workloads.workload("tiny").with_(batch=B, heads=H, head_dim=D, grid=grid)
    inp = workloads.make_integer_inputs(wl)  # integer values: every mean is exact (power-of-two counts aside)
    xc, mean = vsa.cube_permute_pool(to_dev(inp["q"]), grid)
    assert np.array_equal(to_bits(xc), oracle.cube_permute(inp["q"], grid))
    ref = oracle.cube_means(oracle.cube_permute(inp["q"], grid), oracle.valid_rows(grid))
    got = mean.cpu().numpy().astype(np.float64)
    # fp32 means of integer sums divided by the valid count: within one fp32 rounding.
    assert np.abs(got - ref).max() <= 1e-6 * max(1.0, np.abs(ref).max())
