"""Pins of the oracle's linear branch (O6).

References: torch's elu for phi; per-query direct sums written as plain Python
loops over keys (a different association order from the oracle's per-cube
matrix states); closed forms for constant values and for "everything
selected".
"""

import numpy as np
import pytest
import torch

import oracle
import workloads
from tests.test_oracle_permute import reshape_map


def test_phi_is_elu_plus_one():
    x = np.linspace(-30, 30, 1201)
    ref = torch.nn.functional.elu(torch.from_numpy(x), alpha=1.0).numpy() + 1.0
    assert np.abs(oracle.phi(x) - ref).max() < 1e-15
    assert np.all(oracle.phi(x) > 0)


def direct_linear(qf, kf, vf, grid, idx_h):
    """Per-query loops: O = sum_r w_r v_r / sum_r w_r, w_r = phi(q).phi(k_r), r valid & unselected."""
    m = reshape_map(grid)
    cube_of = {}
    for r, s in enumerate(m):
        if s >= 0:
            cube_of[s] = r // 64
    S, D = qf.shape
    out = np.zeros_like(qf)
    pk = [oracle.phi(kf[r]) for r in range(S)]
    for a in range(S):
        sel = set(idx_h[cube_of[a]].tolist())
        pq = oracle.phi(qf[a])
        num = np.zeros(D)
        den = 0.0
        for r in range(S):
            if cube_of[r] in sel:
                continue
            w = float(sum(pq[d] * pk[r][d] for d in range(D)))
            num += w * vf[r]
            den += w
        out[a] = num / den if den > 0 else 0.0
    return out


@pytest.mark.parametrize("grid,topk", [((4, 4, 8), 1), ((5, 6, 7), 2), ((8, 4, 5), 3)])
def test_linear_matches_direct_sums(grid, topk):
    D = 4
    rng = np.random.default_rng(21)
    S = grid[0] * grid[1] * grid[2]
    inp = {n: workloads.round_to_bf16_bits(rng.standard_normal((1, S, 1, D)).astype(np.float32))
           for n in ("q", "k", "v")}
    valid = oracle.valid_rows(grid)
    qc, kc, vc = (oracle.cube_permute(inp[n], grid) for n in ("q", "k", "v"))
    idx = oracle.select_topk(qc, kc, valid, topk)
    lin = oracle.linear_branch(qc, kc, vc, valid, idx)
    lin_tok = oracle.cube_unpermute(lin, grid)[0, :, 0]
    ref = direct_linear(*(oracle.bf16_to_f64(inp[n][0, :, 0]) for n in ("q", "k", "v")), grid, idx[0, 0])
    assert np.abs(lin_tok - ref).max() < 1e-12


def test_linear_all_selected_is_zero_and_constant_v():
    grid = (8, 8, 4)
    rng = np.random.default_rng(22)
    S = 256
    inp = {n: workloads.round_to_bf16_bits(rng.standard_normal((1, S, 2, 8)).astype(np.float32))
           for n in ("q", "k", "v")}
    valid = oracle.valid_rows(grid)
    qc, kc, vc = (oracle.cube_permute(inp[n], grid) for n in ("q", "k", "v"))
    nc = oracle.n_cubes(grid)
    full = oracle.select_topk(qc, kc, valid, nc)
    assert np.all(oracle.linear_branch(qc, kc, vc, valid, full) == 0)
    vconst = np.full_like(vc, workloads.round_to_bf16_bits(np.array([-0.75], np.float32))[0])
    vconst[:, :, ~valid] = 0
    idx = oracle.select_topk(qc, kc, valid, 1)
    lin = oracle.linear_branch(qc, kc, vconst, valid, idx)
    assert np.abs(lin - (-0.75)).max() < 1e-14


def test_linear_weights_exclude_padding():
    # One-cube-row grid 1x1x6 -> 2 cubes, the second with 2 valid tokens.
    # Select cube 0: the linear branch must average only the 2 valid tokens of
    # cube 1, whatever the padded rows hold.
    grid = (1, 1, 6)
    v = np.zeros((1, 6, 1, 1), np.float32)
    v[0, :, 0, 0] = [9, 9, 9, 9, 1.0, 3.0]
    q = np.zeros_like(v)
    k = np.zeros_like(v)
    bits = {n: workloads.round_to_bf16_bits(a) for n, a in (("q", q), ("k", k), ("v", v))}
    valid = oracle.valid_rows(grid)
    qc, kc, vc = (oracle.cube_permute(bits[n], grid) for n in ("q", "k", "v"))
    idx = np.zeros((1, 1, 2, 1), dtype=np.int32)
    lin = oracle.linear_branch(qc, kc, vc, valid, idx)
    # phi(0) = 1 for q and k: equal weights on the two valid tokens of cube 1.
    assert np.all(lin[0, 0, valid, 0] == 2.0)


def test_hybrid_forward_is_sum_of_branches():
    grid = (4, 8, 8)
    rng = np.random.default_rng(23)
    inp = {n: workloads.round_to_bf16_bits(rng.standard_normal((2, 256, 2, 8)).astype(np.float32))
           for n in ("q", "k", "v")}
    o_sparse, idx = oracle.forward(inp["q"], inp["k"], inp["v"], grid, 1)
    o_hyb, idx2 = oracle.forward(inp["q"], inp["k"], inp["v"], grid, 1, linear=True)
    assert np.array_equal(idx, idx2)
    valid = oracle.valid_rows(grid)
    qc, kc, vc = (oracle.cube_permute(inp[n], grid) for n in ("q", "k", "v"))
    lin = oracle.cube_unpermute(oracle.linear_branch(qc, kc, vc, valid, idx), grid)
    assert np.abs(o_hyb - (o_sparse + lin)).max() < 1e-14


@pytest.mark.parametrize("grid,topk", [((4, 4, 8), 1), ((5, 6, 7), 2), ((9, 5, 6), 4)])
def test_state_sums_give_the_linear_branch(grid, topk):
    """phi(Q) S_U / (phi(Q) . z_U) from the exported per-cube states and their
    unselected sums equals linear_branch, which the per-query loops above pin."""
    D = 8
    rng = np.random.default_rng(5)
    S = grid[0] * grid[1] * grid[2]
    inp = {n: workloads.round_to_bf16_bits(rng.standard_normal((2, S, 2, D)).astype(np.float32))
           for n in ("q", "k", "v")}
    valid = oracle.valid_rows(grid)
    qc, kc, vc = (oracle.cube_permute(inp[n], grid) for n in ("q", "k", "v"))
    idx = oracle.select_topk(qc, kc, valid, topk)
    st, z = oracle.linear_cube_states(kc, vc, valid)
    su, zu = oracle.unselected_sums(st, z, idx)
    nc = oracle.n_cubes(grid)
    fq = oracle.phi(oracle.bf16_to_f64(qc)).reshape(2, 2, nc, 64, D)
    num = np.einsum("bhird,bhide->bhire", fq, su)
    den = np.einsum("bhird,bhid->bhir", fq, zu)
    got = (num / den[..., None]).reshape(2, 2, nc * 64, D)
    ref = oracle.linear_branch(qc, kc, vc, valid, idx)
    assert np.abs(got - ref).max() < 1e-12


def test_cube_states_sum_to_the_whole_grid():
    """Summed over all cubes, the states are phi(K)^T V and the column sums of
    phi(K) over every raster token of the grid (padding contributes nothing)."""
    grid, D = (5, 7, 6), 8
    rng = np.random.default_rng(9)
    S = grid[0] * grid[1] * grid[2]
    k = workloads.round_to_bf16_bits(rng.standard_normal((1, S, 1, D)).astype(np.float32))
    v = workloads.round_to_bf16_bits(rng.standard_normal((1, S, 1, D)).astype(np.float32))
    valid = oracle.valid_rows(grid)
    st, z = oracle.linear_cube_states(oracle.cube_permute(k, grid), oracle.cube_permute(v, grid), valid)
    kf = oracle.phi(oracle.bf16_to_f64(k[0, :, 0]))
    vf = oracle.bf16_to_f64(v[0, :, 0])
    assert np.abs(st[0, 0].sum(axis=0) - kf.T @ vf).max() < 1e-10
    assert np.abs(z[0, 0].sum(axis=0) - kf.sum(axis=0)).max() < 1e-10


def test_unselected_sums_of_a_full_selection_are_zero():
    grid, D = (4, 8, 8), 4
    rng = np.random.default_rng(2)
    S = grid[0] * grid[1] * grid[2]
    kc, vc = (oracle.cube_permute(workloads.round_to_bf16_bits(
        rng.standard_normal((1, S, 1, D)).astype(np.float32)), grid) for _ in range(2))
    valid = oracle.valid_rows(grid)
    st, z = oracle.linear_cube_states(kc, vc, valid)
    nc = oracle.n_cubes(grid)
    idx = np.tile(np.arange(nc, dtype=np.int32), (1, 1, nc, 1))
    su, zu = oracle.unselected_sums(st, z, idx)
    assert not su.any() and not zu.any()
