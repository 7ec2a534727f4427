"""Pins of the oracle's cube permutation (convention O1) against an independent map.

The independent map pads the raster grid to multiples of 4 with -1 markers and
splits every axis into (cube, local) with a reshape/transpose, which is how a
4x4x4 tiling reads in index algebra.  A wrong axis order, a swapped
cube/local split or a missing pad fails here.
"""

import numpy as np
import pytest

import oracle
import workloads

GRIDS = [(4, 4, 4), (8, 8, 8), (5, 6, 7), (1, 1, 1), (9, 3, 13), (4, 8, 12), (2, 5, 4)]


def reshape_map(grid):
    """Raster token id at every cube-major row (-1 for padding), via reshape."""
    T, H, W = grid
    Tp, Hp, Wp = [((d + 3) // 4) * 4 for d in grid]
    ids = np.full((Tp, Hp, Wp), -1, dtype=np.int64)
    ids[:T, :H, :W] = np.arange(T * H * W).reshape(T, H, W)
    cubes = ids.reshape(Tp // 4, 4, Hp // 4, 4, Wp // 4, 4).transpose(0, 2, 4, 1, 3, 5)
    return cubes.reshape(-1)


@pytest.mark.parametrize("grid", GRIDS)
def test_permute_matches_reshape_map(grid):
    T, H, W = grid
    S = T * H * W
    B, Hh, D = 2, 3, 4
    rng = np.random.default_rng(1)
    x = rng.integers(1, 60000, size=(B, S, Hh, D)).astype(np.uint16)
    xc = oracle.cube_permute(x, grid)
    m = reshape_map(grid)
    assert xc.shape == (B, Hh, m.size, D)
    for r, s in enumerate(m):
        if s < 0:
            assert np.all(xc[:, :, r] == 0)
        else:
            assert np.array_equal(xc[:, :, r], x[:, s])
    assert np.array_equal(oracle.valid_rows(grid), m >= 0)


@pytest.mark.parametrize("grid", GRIDS)
def test_unpermute_inverts_permute(grid):
    T, H, W = grid
    rng = np.random.default_rng(2)
    x = rng.integers(0, 65536, size=(1, T * H * W, 2, 8)).astype(np.uint16)
    assert np.array_equal(oracle.cube_unpermute(oracle.cube_permute(x, grid), grid), x)


def test_token_row_worked_example():
    # Grid 8x8x8: 2x2x2 cubes.  Token (5, 2, 7) lies in cube (1, 0, 1) -> c = 5,
    # local (1, 2, 3) -> l = 1*16 + 2*4 + 3 = 27.
    assert oracle.token_row(5, 2, 7, (8, 8, 8)) == (5, 27)
    # Padded grid 21x45x80 -> 24x48x80: cubes per axis 6, 12, 20.
    assert oracle.cube_grid((21, 45, 80)) == (6, 12, 20)
    assert oracle.n_cubes((21, 45, 80)) == 1440
    # Last token (20, 44, 79): cube (5, 11, 19) -> (5*12 + 11)*20 + 19 = 1439,
    # local (0, 0, 3) -> 3.
    assert oracle.token_row(20, 44, 79, (21, 45, 80)) == (1439, 3)


@pytest.mark.parametrize("name", list(workloads.WORKLOADS))
def test_workload_geometry(name):
    wl = workloads.workload(name)
    assert oracle.n_cubes(wl.grid) == wl.n_cubes
    assert oracle.padded_grid(wl.grid) == wl.padded_grid


def test_720p_every_cube_has_valid_tokens():
    v = oracle.valid_rows((21, 45, 80)).reshape(-1, 64)
    counts = v.sum(axis=1)
    assert counts.min() >= 4
    assert set(np.unique(counts)) <= {4, 16, 64}
    assert v.sum() == 21 * 45 * 80


# ---------------------------------------------------------------- O12 layouts

@pytest.mark.parametrize("grid", GRIDS + [(21, 45, 20), (6, 7, 5)])
def test_compact_rows_are_the_valid_rows_first(grid):
    # Independent construction: the O1 rows of each cube, split by the valid
    # mask with a boolean selection (valid ones first, in row order, then the
    # zero pads).
    T, H, W = grid
    rng = np.random.default_rng(3)
    x = rng.integers(1, 60000, size=(2, T * H * W, 2, 3)).astype(np.uint16)
    xc = oracle.cube_permute(x, grid)
    valid = oracle.valid_rows(grid)
    got = oracle.cube_permute_compact(x, grid)
    for c in range(oracle.n_cubes(grid)):
        rows = xc[:, :, 64 * c:64 * c + 64]
        v = valid[64 * c:64 * c + 64]
        n = int(v.sum())
        assert np.array_equal(got[:, :, 64 * c:64 * c + n], rows[:, :, v])
        assert np.all(got[:, :, 64 * c + n:64 * c + 64] == 0)
    order = oracle.compact_order(grid)
    assert all(sorted(order[c]) == list(range(64)) for c in range(order.shape[0]))


def test_compact_equals_o1_order_on_full_grids():
    x = np.random.default_rng(4).integers(0, 65536, size=(1, 8 * 4 * 12, 2, 4)).astype(np.uint16)
    assert np.array_equal(oracle.cube_permute_compact(x, (8, 4, 12)), oracle.cube_permute(x, (8, 4, 12)))


def test_compact_worked_example():
    # Grid 4x5x4: cubes (0,0,0) full and (0,1,0) with one valid y row (y = 4).
    # Its valid tokens (t, 4, x) in raster order sit at compact rows t*4 + x;
    # token (1, 4, 2) is raster token (1*5 + 4)*4 + 2 = 38, compact row
    # 64 + 6.  Its O1 local index is (1*4 + 0)*4 + 2 = 18.
    grid = (4, 5, 4)
    x = np.zeros((1, 80, 1, 1), dtype=np.uint16)
    x[0, 38, 0, 0] = 777
    assert oracle.cube_permute(x, grid)[0, 0, 64 + 18, 0] == 777
    xc = oracle.cube_permute_compact(x, grid)
    assert xc[0, 0, 64 + 6, 0] == 777 and int((xc != 0).sum()) == 1
    assert list(oracle.compact_order(grid)[1, :16]) == [0, 1, 2, 3, 16, 17, 18, 19, 32, 33, 34, 35, 48, 49, 50, 51]


def test_slots_layout_index_map():
    grid = (5, 6, 7)
    rng = np.random.default_rng(5)
    x = rng.integers(1, 60000, size=(1, 5 * 6 * 7, 2, 8)).astype(np.uint16)
    xc = oracle.cube_permute_compact(x, grid)
    sl = oracle.cube_slots(xc)
    nc = oracle.n_cubes(grid)
    assert sl.shape == (1, 2, nc, 4, 8, 16)
    # Slot-major, each 16-row slot transposed: a reshape/transpose of the rows.
    ref = xc.reshape(1, 2, nc, 4, 16, 8).transpose(0, 1, 2, 3, 5, 4)
    assert np.array_equal(sl, ref)
