"""Pins of the oracle's sliding-tile block lists (O8), independent of its code.

The pages name sliding-tile attention (FastVideo attention-backend article,
item "SLIDING_TILE_ATTN" and the figure comparing NATTEN, Tiled NATTEN and
STA) without a window definition; the reading pinned here is a window of
(wt, wh, ww) key cubes, centred on the query cube where possible and shifted
inwards at the borders.  The brute-force check below restates that reading as
a search over all admissible windows, not as the oracle's formula.
"""

import itertools

import numpy as np
import pytest

import oracle

GRIDS = [(8, 8, 8), (16, 28, 52), (5, 6, 7), (4, 4, 4), (12, 4, 20), (24, 13, 9)]
WINDOWS = [(1, 1, 1), (3, 3, 3), (2, 4, 3), (3, 5, 7), (5, 5, 5), (9, 9, 9), (1, 2, 1)]


def cube_coords(j, cg):
    ct, ch, cw = cg
    return j // (ch * cw), (j // cw) % ch, j % cw


def brute_axis(c, n, w):
    """All windows [s, s + w) inside [0, n) that hold c; keep the one whose
    centre s + (w - 1) / 2 is nearest to c, the higher start on a tie."""
    if w >= n:
        return set(range(n))
    cands = [s for s in range(0, n - w + 1) if s <= c < s + w]
    best = min(cands, key=lambda s: (abs(2 * s + w - 1 - 2 * c), -s))
    return set(range(best, best + w))


@pytest.mark.parametrize("grid", GRIDS)
@pytest.mark.parametrize("window", WINDOWS)
def test_sta_index_matches_brute_force(grid, window):
    cg = oracle.cube_grid(grid)
    nc = oracle.n_cubes(grid)
    idx = oracle.sta_index(grid, window)
    k = int(np.prod([min(w, n) for w, n in zip(window, cg)]))
    assert idx.shape == (nc, k) and idx.dtype == np.int32
    for i in range(nc):
        t, y, x = cube_coords(i, cg)
        want = [j for j in range(nc)
                if cube_coords(j, cg)[0] in brute_axis(t, cg[0], window[0])
                and cube_coords(j, cg)[1] in brute_axis(y, cg[1], window[1])
                and cube_coords(j, cg)[2] in brute_axis(x, cg[2], window[2])]
        assert list(idx[i]) == want  # brute force lists j ascending


def test_window_one_is_the_own_cube():
    idx = oracle.sta_index((16, 28, 52), (1, 1, 1))
    assert np.array_equal(idx[:, 0], np.arange(idx.shape[0]))


def test_window_covering_the_grid_is_dense():
    grid = (12, 4, 20)
    nc = oracle.n_cubes(grid)
    idx = oracle.sta_index(grid, (9, 9, 9))
    assert np.array_equal(idx, np.tile(np.arange(nc, dtype=np.int32), (nc, 1)))


def test_interior_odd_window_is_a_box_around_the_query():
    grid, window = (21, 45, 80), (3, 5, 7)
    cg = oracle.cube_grid(grid)
    idx = oracle.sta_index(grid, window)
    r = [w // 2 for w in window]
    for t, y, x in itertools.product(range(r[0], cg[0] - r[0]), range(r[1], cg[1] - r[1]),
                                     range(r[2], cg[2] - r[2])):
        i = (t * cg[1] + y) * cg[2] + x
        box = sorted((tt * cg[1] + yy) * cg[2] + xx
                     for tt in range(t - r[0], t + r[0] + 1)
                     for yy in range(y - r[1], y + r[1] + 1)
                     for xx in range(x - r[2], x + r[2] + 1))
        assert list(idx[i]) == box


def test_border_windows_are_flush_and_hold_the_query():
    grid, window = (16, 28, 52), (3, 3, 5)
    cg = oracle.cube_grid(grid)
    idx = oracle.sta_index(grid, window)
    for i in range(idx.shape[0]):
        assert i in idx[i]
        coords = np.array([cube_coords(int(j), cg) for j in idx[i]])
        for a in range(3):
            lo, hi = coords[:, a].min(), coords[:, a].max()
            assert hi - lo + 1 == min(window[a], cg[a])
            assert lo >= 0 and hi < cg[a]
    # first and last cube of the grid: windows flush against the borders
    assert list(idx[0]) == sorted((tt * cg[1] + yy) * cg[2] + xx for tt in range(3) for yy in range(3)
                                  for xx in range(5))
    last = idx.shape[0] - 1
    assert list(idx[last]) == sorted((tt * cg[1] + yy) * cg[2] + xx for tt in range(cg[0] - 3, cg[0])
                                     for yy in range(cg[1] - 3, cg[1]) for xx in range(cg[2] - 5, cg[2]))
