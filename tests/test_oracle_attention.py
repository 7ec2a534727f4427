"""Pins of the oracle's fine stage (O5) and whole forward (O7).

Independent references: torch's scaled_dot_product_attention on CPU float64
(dense, or with an explicit token-level boolean block mask built from the
reshape map), closed forms, and the row-stochastic property.
"""

import math

import numpy as np
import pytest
import torch

import oracle
import workloads
from tests.test_oracle_permute import reshape_map


def sdpa_f64(q, k, v, scale, mask=None):
    """torch SDPA in float64 on [S, D] per head; mask [Sq, Sk] bool (True = attend)."""
    qt = torch.from_numpy(q)[None]
    kt = torch.from_numpy(k)[None]
    vt = torch.from_numpy(v)[None]
    m = None if mask is None else torch.from_numpy(mask)[None]
    return torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=m, scale=scale)[0].numpy()


def rand_inputs(grid, B, Hh, D, seed):
    rng = np.random.default_rng(seed)
    S = grid[0] * grid[1] * grid[2]
    return {n: workloads.round_to_bf16_bits(rng.standard_normal((B, S, Hh, D)).astype(np.float32))
            for n in ("q", "k", "v")}


@pytest.mark.parametrize("grid", [(4, 4, 4), (8, 8, 8), (5, 6, 7), (3, 9, 5)])
def test_all_cubes_selected_is_dense_attention(grid):
    D = 16
    inp = rand_inputs(grid, 1, 2, D, 11)
    nc = oracle.n_cubes(grid)
    scale = 1.0 / math.sqrt(D)
    out, idx = oracle.forward(inp["q"], inp["k"], inp["v"], grid, nc, scale)
    assert np.array_equal(idx[0, 0, 0], np.arange(nc))
    for h in range(2):
        q, k, v = (oracle.bf16_to_f64(inp[n][0, :, h]) for n in ("q", "k", "v"))
        ref = sdpa_f64(q, k, v, scale)
        assert np.abs(out[0, :, h] - ref).max() < 1e-12


@pytest.mark.parametrize("grid,topk", [((8, 8, 8), 2), ((5, 6, 7), 3), ((9, 5, 6), 1)])
def test_block_mask_matches_masked_sdpa(grid, topk):
    # Token-level mask: query token a attends key token b iff b's cube is in the
    # selected list of a's cube.  Cube membership comes from the reshape map.
    D = 8
    inp = rand_inputs(grid, 1, 2, D, 12)
    scale = 0.3
    out, idx = oracle.forward(inp["q"], inp["k"], inp["v"], grid, topk, scale)
    m = reshape_map(grid)
    cube_of = np.empty(grid[0] * grid[1] * grid[2], dtype=np.int64)
    for r, s in enumerate(m):
        if s >= 0:
            cube_of[s] = r // 64
    for h in range(2):
        sel = [set(idx[0, h, i].tolist()) for i in range(oracle.n_cubes(grid))]
        mask = np.array([[cube_of[b] in sel[cube_of[a]] for b in range(cube_of.size)]
                         for a in range(cube_of.size)])
        q, k, v = (oracle.bf16_to_f64(inp[n][0, :, h]) for n in ("q", "k", "v"))
        ref = sdpa_f64(q, k, v, scale, mask)
        assert np.abs(out[0, :, h] - ref).max() < 1e-12


def test_rows_are_stochastic_and_zero_off_valid_keys():
    grid = (5, 6, 7)
    inp = rand_inputs(grid, 1, 1, 16, 13)
    valid = oracle.valid_rows(grid)
    qc = oracle.cube_permute(inp["q"], grid)
    kc = oracle.cube_permute(inp["k"], grid)
    vc = oracle.cube_permute(inp["v"], grid)
    cubes = [0, 3, 5]
    _, lse, p = oracle.attention_cube(qc[0, 0, 64:128], kc[0, 0], vc[0, 0], valid, cubes, 0.25,
                                      return_probs=True)
    keys = np.array([64 * j + l for j in cubes for l in range(64)])
    assert np.all(p >= 0)
    assert np.abs(p.sum(axis=1) - 1).max() < 1e-12
    assert np.all(p[:, ~valid[keys]] == 0)
    # lse against torch.logsumexp of the valid scaled logits.
    q = oracle.bf16_to_f64(qc[0, 0, 64:128])
    k = oracle.bf16_to_f64(kc[0, 0, keys[valid[keys]]])
    ref = torch.logsumexp(torch.from_numpy(0.25 * q @ k.T), dim=1).numpy()
    assert np.abs(lse - ref).max() < 1e-12


def test_constant_values_give_constant_output():
    grid = (8, 4, 6)
    inp = rand_inputs(grid, 1, 2, 8, 14)
    inp["v"][:] = workloads.round_to_bf16_bits(np.full(inp["v"].shape, 1.375, np.float32))
    out, _ = oracle.forward(inp["q"], inp["k"], inp["v"], grid, 2)
    assert np.abs(out - 1.375).max() < 1e-14


def test_zero_queries_average_valid_values():
    # q = 0: uniform weights over the valid keys of the selected cubes.  On a
    # one-cube grid of 2 tokens the output is the mean of the 2 value rows.
    grid = (1, 1, 2)
    v = np.array([[[[1.0, 2.0]], [[3.0, -6.0]]]], dtype=np.float32)  # [1, 2, 1, 2]
    bits = workloads.round_to_bf16_bits(v)
    q = np.zeros_like(bits)
    out, _ = oracle.forward(q, bits, bits, grid, 1)
    assert np.array_equal(out[0, :, 0], np.array([[2.0, -2.0], [2.0, -2.0]]))


def test_own_cube_only_is_local_dense_attention():
    grid = (8, 8, 8)
    inp = rand_inputs(grid, 1, 1, 32, 15)
    nc = oracle.n_cubes(grid)
    idx = np.arange(nc, dtype=np.int32).reshape(1, 1, nc, 1)
    valid = oracle.valid_rows(grid)
    qc, kc, vc = (oracle.cube_permute(inp[n], grid) for n in ("q", "k", "v"))
    o, _ = oracle.sparse_attention(qc, kc, vc, valid, idx, 0.2)
    for i in range(nc):
        rows = slice(64 * i, 64 * i + 64)
        ref = sdpa_f64(*(oracle.bf16_to_f64(x[0, 0, rows]) for x in (qc, kc, vc)), 0.2)
        assert np.abs(o[0, 0, rows] - ref).max() < 1e-12
