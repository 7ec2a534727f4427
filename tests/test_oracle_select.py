"""Pins of the oracle's coarse stage: cube means (O2), block scores (O3), top-k (O4)."""

import numpy as np
import pytest

import oracle
import workloads


def brute_topk(scores, k):
    """Python-tuple sort: best score first, lower index first among equals."""
    order = sorted(range(len(scores)), key=lambda j: (-float(scores[j]), j))
    return sorted(order[:k])


def test_topk_row_brute_force():
    rng = np.random.default_rng(3)
    for trial in range(200):
        n = int(rng.integers(1, 40))
        k = int(rng.integers(1, n + 1))
        # Coarse integer values produce many exact ties.
        s = rng.integers(-3, 4, size=n).astype(np.float64)
        assert list(oracle.topk_row(s, k)) == brute_topk(s, k)


def test_topk_signed_zero_ties():
    s = np.array([1.0, -0.0, 0.0, -0.0, 2.0])
    # Best is index 4, then index 0, then the zeros tie: lowest index 1 wins.
    assert list(oracle.topk_row(s, 3)) == [0, 1, 4]


def test_topk_output_ascending_not_by_score():
    s = np.array([0.5, 3.0, 1.0, 2.0])
    assert list(oracle.topk_row(s, 3)) == [1, 2, 3]


def test_cube_means_ignore_padding():
    # Grid 2x3x5 -> padded 4x4x8, 2 cubes; each cube has a constant value on its
    # valid tokens.  The mean must be that constant, not diluted by zero pads.
    grid = (2, 3, 5)
    valid = oracle.valid_rows(grid)
    T, H, W = grid
    x = np.zeros((1, T * H * W, 1, 2))
    for t in range(T):
        for y in range(H):
            for xx in range(W):
                c, _ = oracle.token_row(t, y, xx, grid)
                x[0, (t * H + y) * W + xx, 0] = [3.0, -1.5] if c == 0 else [0.25, 7.0]
    xc = oracle.cube_permute(x, grid)
    m = oracle.cube_means(xc, valid)
    assert np.array_equal(m[0, 0], np.array([[3.0, -1.5], [0.25, 7.0]]))


def test_worked_example_three_cubes():
    # Grid 4x4x12: cubes 0, 1, 2 along x.  Query cube i has constant q = i + 1
    # in dimension 0; key cube j has constant k = (2, -1, 2)[j] in dimension 0.
    # Scores s_ij = (i + 1) * k_j: every row ranks cubes 0 and 2 equal (tie ->
    # lower index 0 first), then cube 1.
    grid = (4, 4, 12)
    valid = oracle.valid_rows(grid)
    xc_q = np.zeros((1, 1, 192, 2))
    xc_k = np.zeros((1, 1, 192, 2))
    for c, kv in enumerate([2.0, -1.0, 2.0]):
        xc_q[0, 0, 64 * c:64 * c + 64, 0] = c + 1
        xc_k[0, 0, 64 * c:64 * c + 64, 0] = kv
    s = oracle.block_scores(oracle.cube_means(xc_q, valid), oracle.cube_means(xc_k, valid))
    assert np.array_equal(s[0, 0], np.array([[2.0, -1.0, 2.0], [4.0, -2.0, 4.0], [6.0, -3.0, 6.0]]))
    idx1 = oracle.select_topk(xc_q, xc_k, valid, 1)
    assert idx1[0, 0, :, 0].tolist() == [0, 0, 0]
    idx2 = oracle.select_topk(xc_q, xc_k, valid, 2)
    assert idx2[0, 0].tolist() == [[0, 2]] * 3


def test_select_full_and_zero_keys():
    wl = workloads.workload("tiny")
    inp = workloads.make_tie_inputs(wl, "zero_k")
    valid = oracle.valid_rows(wl.grid)
    qc = oracle.cube_permute(inp["q"], wl.grid)
    kc = oracle.cube_permute(inp["k"], wl.grid)
    idx = oracle.select_topk(qc, kc, valid, 3)
    assert np.array_equal(idx, np.broadcast_to(np.arange(3, dtype=np.int32), idx.shape))
    full = oracle.select_topk(qc, kc, valid, wl.n_cubes)
    assert np.array_equal(full, np.broadcast_to(np.arange(wl.n_cubes, dtype=np.int32), full.shape))


def test_select_brute_force_from_raw_tokens():
    # Recompute the pooled scores straight from raster tokens (cube membership
    # from the reshape map in the permutation pins) and rank them by brute force.
    from tests.test_oracle_permute import reshape_map

    grid = (5, 6, 9)
    rng = np.random.default_rng(5)
    T, H, W = grid
    S = T * H * W
    q = workloads.round_to_bf16_bits(rng.standard_normal((1, S, 2, 8)).astype(np.float32))
    k = workloads.round_to_bf16_bits(rng.standard_normal((1, S, 2, 8)).astype(np.float32))
    qf = workloads.bf16_bits_to_f32(q).astype(np.float64)
    kf = workloads.bf16_bits_to_f32(k).astype(np.float64)
    m = reshape_map(grid).reshape(-1, 64)
    nc = m.shape[0]
    valid = oracle.valid_rows(grid)
    qc = oracle.cube_permute(q, grid)
    kc = oracle.cube_permute(k, grid)
    for kk in (1, 3, nc):
        idx = oracle.select_topk(qc, kc, valid, kk)
        for h in range(2):
            qbar = [qf[0, [s for s in m[c] if s >= 0], h].mean(axis=0) for c in range(nc)]
            kbar = [kf[0, [s for s in m[c] if s >= 0], h].mean(axis=0) for c in range(nc)]
            for i in range(nc):
                sc = [float(np.dot(qbar[i], kbar[j])) for j in range(nc)]
                assert idx[0, h, i].tolist() == brute_topk(sc, kk)


def test_integer_inputs_give_exact_scores():
    wl = workloads.workload("tiny")
    inp = workloads.make_integer_inputs(wl)
    valid = oracle.valid_rows(wl.grid)
    qb = oracle.cube_means(oracle.cube_permute(inp["q"], wl.grid), valid)
    kb = oracle.cube_means(oracle.cube_permute(inp["k"], wl.grid), valid)
    s = oracle.block_scores(qb, kb)
    # Means are multiples of 1/64, so scores are multiples of 2^-12.
    assert np.array_equal(s * 4096, np.round(s * 4096))
    assert np.abs(s).max() < 2 ** 11


@pytest.mark.parametrize("name", ["tiny", "wan1.3b", "wan14b", "720p", "hybrid"])
def test_kept_fraction_matches_sparsity(name):
    # The pages: kept fraction = 1 - sparsity (golden file lists the cited values).
    wl = workloads.workload(name)
    k = workloads.topk_for_sparsity(wl.sparsity, wl.n_cubes)
    assert k == wl.topk
    frac = k / wl.n_cubes
    assert 1 - wl.sparsity - 1e-12 <= frac < 1 - wl.sparsity + 1.0 / wl.n_cubes


def test_golden_sparsity_fractions():
    import os

    path = os.path.join(os.path.dirname(__file__), "golden", "sparsity_kept_fraction.txt")
    rows = [ln.split("#")[0].split() for ln in open(path, encoding="utf-8")]
    rows = [r for r in rows if r]
    assert rows
    for s, lo, hi in rows:
        s, lo, hi = float(s), float(lo), float(hi)
        for nc in (8, 364, 455, 1440):
            frac = workloads.topk_for_sparsity(s, nc) / nc
            assert lo - 1e-12 <= frac < hi + 1.0 / nc
