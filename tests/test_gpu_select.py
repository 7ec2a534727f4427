"""GPU parity: coarse stage (cube means, block scores, top-k).

Bit-exact on integer-valued inputs (all fp32 sums exact on both sides, exact
ties resolved to the lower cube index); on float inputs every GPU row must be
a valid top-k of the oracle's fp64 scores up to a relative 1e-5 near-tie band.
"""

import numpy as np
import pytest

import oracle
import workloads
from tests.gpu_util import to_bits, to_dev, topk_valid_under

pytestmark = pytest.mark.gpu


def run_select(inp, wl, topk):
    import block_sparse_video_cube_amd as vsa

    qc = vsa.cube_permute(to_dev(inp["q"]), wl.grid)
    kc = vsa.cube_permute(to_dev(inp["k"]), wl.grid)
    return vsa.select_topk(qc, kc, wl.grid, topk).cpu().numpy()


def oracle_select(inp, wl, topk):
    valid = oracle.valid_rows(wl.grid)
    qc = oracle.cube_permute(inp["q"], wl.grid)
    kc = oracle.cube_permute(inp["k"], wl.grid)
    return oracle.select_topk(qc, kc, valid, topk)


# Grids whose per-axis remainders give power-of-two valid counts per cube, so
# integer-valued means stay exact in fp32.
INT_CASES = [
    ("tiny", None, None),
    ("tiny", (8, 8, 8), 1),
    ("tiny", (8, 8, 8), 8),
    ("tiny", (9, 6, 12), 5),     # valid counts 1, 2, 4 per axis
    ("tiny", (16, 12, 20), 17),  # 60 cubes
    ("tiny", (4, 4, 260), 20),   # 65 cubes: two 64-wide lanes passes
]


@pytest.mark.parametrize("name,grid,topk", INT_CASES)
@pytest.mark.parametrize("D", [64, 128])
def test_topk_bit_exact_integer_inputs(name, grid, topk, D):
    wl = workloads.workload(name).with_(head_dim=D)
    if grid is not None:
        wl = wl.with_(grid=grid)
    if topk is not None:
        wl = wl.with_(topk=topk)
    inp = workloads.make_integer_inputs(wl)
    got = run_select(inp, wl, wl.topk)
    ref = oracle_select(inp, wl, wl.topk)
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("kind", ["zero_k", "periodic_k"])
@pytest.mark.parametrize("grid,topk", [((8, 8, 8), 3), ((8, 8, 32), 7), ((4, 8, 64), 13)])
def test_topk_bit_exact_tie_cases(kind, grid, topk):
    wl = workloads.workload("tiny").with_(grid=grid, topk=topk)
    inp = workloads.make_tie_inputs(wl, kind)
    got = run_select(inp, wl, topk)
    ref = oracle_select(inp, wl, topk)
    assert np.array_equal(got, ref)


def test_topk_integer_720p_shape_two_heads():
    # 1440 cubes, partial cubes with 4 / 16 valid tokens: exact on both sides.
    wl = workloads.workload("720p").with_(heads=2)
    inp = workloads.make_integer_inputs(wl)
    got = run_select(inp, wl, wl.topk)
    ref = oracle_select(inp, wl, wl.topk)
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("name", ["wan1.3b", "wan14b"])
def test_topk_integer_wan_shapes_two_heads(name):
    # 364 and 455 cubes (12 and 15 score tiles of 32, the last one ragged),
    # both entry points.
    import block_sparse_video_cube_amd as vsa

    wl = workloads.workload(name).with_(heads=2)
    inp = workloads.make_integer_inputs(wl)
    ref = oracle_select(inp, wl, wl.topk)
    assert np.array_equal(run_select(inp, wl, wl.topk), ref)
    _, qbar = vsa.cube_permute_pool(to_dev(inp["q"]), wl.grid)
    _, kbar = vsa.cube_permute_pool(to_dev(inp["k"]), wl.grid)
    assert np.array_equal(vsa.select_topk_pooled(qbar, kbar, wl.grid, wl.topk).cpu().numpy(), ref)


@pytest.mark.parametrize("grid,topk", [((8, 8, 8), 2), ((5, 6, 7), 3), ((13, 10, 22), 9)])
def test_topk_float_inputs_near_tie_valid(grid, topk):
    wl = workloads.workload("tiny").with_(grid=grid, topk=topk, heads=3)
    inp = workloads.make_inputs(wl)
    got = run_select(inp, wl, topk)
    valid = oracle.valid_rows(wl.grid)
    qb = oracle.cube_means(oracle.cube_permute(inp["q"], wl.grid), valid)
    kb = oracle.cube_means(oracle.cube_permute(inp["k"], wl.grid), valid)
    s = oracle.block_scores(qb, kb)
    ref = oracle.select_topk(oracle.cube_permute(inp["q"], wl.grid), oracle.cube_permute(inp["k"], wl.grid),
                             valid, topk)
    exact = 0
    for h in range(wl.heads):
        for i in range(wl.n_cubes):
            assert topk_valid_under(s[0, h, i], got[0, h, i], topk)
            exact += int(np.array_equal(got[0, h, i], ref[0, h, i]))
    print(f"rows identical to the oracle: {exact}/{wl.heads * wl.n_cubes}")


@pytest.mark.parametrize("name,grid,topk", INT_CASES)
def test_pooled_path_matches_oracle_integer_inputs(name, grid, topk):
    import block_sparse_video_cube_amd as vsa

    wl = workloads.workload(name).with_(head_dim=128)
    if grid is not None:
        wl = wl.with_(grid=grid)
    if topk is not None:
        wl = wl.with_(topk=topk)
    inp = workloads.make_integer_inputs(wl)
    _, qbar = vsa.cube_permute_pool(to_dev(inp["q"]), wl.grid)
    _, kbar = vsa.cube_permute_pool(to_dev(inp["k"]), wl.grid)
    got = vsa.select_topk_pooled(qbar, kbar, wl.grid, wl.topk).cpu().numpy()
    assert np.array_equal(got, oracle_select(inp, wl, wl.topk))
