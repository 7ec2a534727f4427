"""GPU parity: coarse stage (cube means, block scores, top-k).

Bit-exact on integer-valued inputs (all fp32 sums exact on both sides, exact
ties resolved to the lower cube index); on float inputs every GPU row must be
a valid top-k of the oracle's fp64 scores up to a relative 1e-5 near-tie band.
Crafted score rows (exactly representable) put 1 to 90 keys in the 16-bit
bucket of the k-th largest score, with and without ties, so that both paths
of the top-k search (bucket compacted to one key per lane, or searched over
all keys) are checked against the oracle bit for bit.
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


FLOAT_GRIDS = [((8, 8, 8), 2), ((5, 6, 7), 3), ((13, 10, 22), 9), ((21, 45, 20), 30)]


@pytest.mark.parametrize("grid,topk", FLOAT_GRIDS)
@pytest.mark.parametrize("D", [64, 128])
def test_pooled_topk_float_inputs_near_tie_valid(grid, topk, D):
    # The benchmark's chain: means of Q from vsa_cube_pool, of K from
    # vsa_cube_permute_pool, then vsa_select_topk_pooled; on float inputs and
    # partial cubes with non-power-of-two valid counts (5 x 6 x 7: counts
    # 1..3 per axis).
    import block_sparse_video_cube_amd as vsa

    wl = workloads.workload("tiny").with_(grid=grid, topk=topk, heads=3, head_dim=D)
    inp = workloads.make_inputs(wl)
    qbar = vsa.cube_pool(to_dev(inp["q"]), wl.grid)
    _, kbar = vsa.cube_permute_pool(to_dev(inp["k"]), wl.grid)
    got = vsa.select_topk_pooled(qbar, kbar, wl.grid, topk).cpu().numpy()
    valid = oracle.valid_rows(wl.grid)
    qc, kc = oracle.cube_permute(inp["q"], wl.grid), oracle.cube_permute(inp["k"], wl.grid)
    s = oracle.block_scores(oracle.cube_means(qc, valid), oracle.cube_means(kc, valid))
    ref = oracle.select_topk(qc, kc, valid, topk)
    exact = 0
    for h in range(wl.heads):
        for i in range(wl.n_cubes):
            assert topk_valid_under(s[0, h, i], got[0, h, i], topk), (h, i)
            exact += int(np.array_equal(got[0, h, i], ref[0, h, i]))
    print(f"pooled rows identical to the oracle: {exact}/{wl.heads * wl.n_cubes}")


@pytest.mark.parametrize("grid", [(5, 6, 7), (13, 10, 22), (8, 8, 8)])
@pytest.mark.parametrize("D", [64, 128])
def test_cube_means_identical_across_entry_points(grid, D):
    # vsa_select_topk pools cube-major rows itself (its workspace starts with
    # the Q means, then the K means); vsa_cube_permute_pool and vsa_cube_pool
    # pool raster rows.  All three sum in the same order, so the means and the
    # selections agree bit for bit on float inputs.
    import torch

    import block_sparse_video_cube_amd as vsa

    wl = workloads.workload("tiny").with_(grid=grid, heads=2, head_dim=D, topk=3)
    inp = workloads.make_inputs(wl)
    q, k = to_dev(inp["q"]), to_dev(inp["k"])
    qc, qbar = vsa.cube_permute_pool(q, wl.grid)
    kc, kbar = vsa.cube_permute_pool(k, wl.grid)
    assert torch.equal(vsa.cube_pool(q, wl.grid), qbar)
    g = vsa.make_geom(wl.batch, wl.heads, D, wl.grid)
    ws = torch.empty(vsa.workspace_bytes(g), dtype=torch.uint8, device="cuda:0")
    idx = vsa.select_topk(qc, kc, wl.grid, wl.topk, workspace=ws)
    torch.cuda.synchronize()
    n = qbar.numel()
    means = ws[:8 * n].view(torch.float32)
    assert torch.equal(means[:n].view_as(qbar), qbar)
    assert torch.equal(means[n:].view_as(kbar), kbar)
    assert torch.equal(vsa.select_topk_pooled(qbar, kbar, wl.grid, wl.topk), idx)


# Crafted scores through vsa_select_topk_pooled: with qbar = e0 every score
# row is kbar[:, 0] exactly (fp32 products by 1).  A cluster of keys shares
# the upper 16 bits of the k-th largest score (values 1 + 8 j ulp apart), the
# rest lie far below or above it.  The search compacts that bucket when it
# holds at most 64 keys and searches all keys otherwise; both must give the
# oracle's rows, ties to the lower index included.
@pytest.mark.parametrize("bucket,above,ties", [(63, 10, False), (64, 10, False), (65, 10, False), (90, 30, False),
                                               (64, 0, True), (70, 5, True), (1, 40, False)])
def test_topk_bucket_sizes_around_64(bucket, above, ties):
    import torch

    import block_sparse_video_cube_amd as vsa

    grid, D, nc = (16, 32, 32), 64, 256
    assert oracle.n_cubes(grid) == nc
    rng = np.random.default_rng(bucket * 7 + above)
    perm = rng.permutation(nc)
    s = np.full(nc, 0.5, dtype=np.float32)
    s[perm[:above]] = 2.0 + np.arange(above, dtype=np.float32)            # clearly above the bucket
    cluster = perm[above:above + bucket]
    if ties:
        s[cluster] = np.float32(1.0) + np.float32(2.0 ** -20) * (np.arange(bucket) // 4).astype(np.float32)
    else:
        s[cluster] = np.float32(1.0) + np.float32(2.0 ** -20) * np.arange(bucket, dtype=np.float32)
    kbar = np.zeros((1, 1, nc, D), dtype=np.float32)
    kbar[0, 0, :, 0] = s
    qbar = np.zeros((1, 1, nc, D), dtype=np.float32)
    qbar[0, 0, :, 0] = 1.0
    for topk in sorted({above + 1, above + bucket // 2, above + bucket, min(nc, above + bucket + 3)}):
        got = vsa.select_topk_pooled(torch.from_numpy(qbar).to("cuda:0"), torch.from_numpy(kbar).to("cuda:0"),
                                     grid, topk).cpu().numpy()
        want = oracle.topk_row(s.astype(np.float64), topk)
        assert np.all(got[0, 0] == want[None, :]), (bucket, above, ties, topk)
