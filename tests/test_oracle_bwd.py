"""Pins of the oracle's fine-stage backward (O9), independent of its code.

- torch autograd (CPU, float64) through a dense token-level masked softmax
  attention built from the block list: a library's chain rule, not the
  oracle's formula;
- central finite differences of the scalar loss sum(O * dO) in float64;
- closed forms: V constant gives dQ = dK = 0; the dK rows of a head sum to 0
  (every softmax row's dS sums to 0); the dV rows sum to the sum of dO rows.
"""

import math

import numpy as np
import pytest
import torch

import oracle
import workloads

CASES = [
    # (grid, D, k)
    ((8, 8, 8), 16, 2),
    ((5, 6, 7), 8, 3),     # partial cubes: padded keys and queries
    ((4, 8, 12), 16, 6),   # k = Nc: dense
]


def inputs(grid, D, k, seed, H=2):
    wl = workloads.workload("tiny").with_(heads=H, head_dim=D, grid=grid, topk=k, seed=seed)
    inp = workloads.make_inputs(wl)
    rng = np.random.default_rng(seed + 1)
    do = rng.standard_normal(inp["q"].shape)
    valid = oracle.valid_rows(grid)
    qc, kc = oracle.cube_permute(inp["q"], grid), oracle.cube_permute(inp["k"], grid)
    idx = oracle.select_topk(qc, kc, valid, k)
    return inp, do, idx


def torch_dense_grads(q, k, v, do, grid, idx, scale):
    """Autograd through softmax(scale q k^T + mask) v over raster tokens."""
    B, S, H, D = q.shape
    T, Hg, W = grid
    cube_of = np.empty(S, dtype=np.int64)
    for s in range(S):
        t, y, x = s // (Hg * W), (s // W) % Hg, s % W
        cube_of[s] = oracle.token_row(t, y, x, grid)[0]
    grads = [np.zeros((B, S, H, D)) for _ in range(3)]
    for b in range(B):
        for h in range(H):
            allowed = np.zeros((S, S), dtype=bool)
            for r in range(S):
                allowed[r] = np.isin(cube_of, idx[b, h, cube_of[r]])
            mask = torch.from_numpy(np.where(allowed, 0.0, -np.inf))
            tq, tk, tv = (torch.tensor(oracle.bf16_to_f64(x[b, :, h]), requires_grad=True) for x in (q, k, v))
            o = torch.softmax(scale * tq @ tk.T + mask, dim=-1) @ tv
            (o * torch.from_numpy(do[b, :, h])).sum().backward()
            for g, t in zip(grads, (tq, tk, tv)):
                g[b, :, h] = t.grad.numpy()
    return grads


@pytest.mark.parametrize("grid,D,k", CASES)
def test_backward_matches_torch_autograd(grid, D, k):
    inp, do, idx = inputs(grid, D, k, 31)
    scale = 1.0 / math.sqrt(D)
    got = oracle.backward(inp["q"], inp["k"], inp["v"], do, grid, idx, scale)
    ref = torch_dense_grads(inp["q"], inp["k"], inp["v"], do, grid, idx, scale)
    for name, g, r in zip("qkv", got, ref):
        assert np.abs(g - r).max() <= 1e-10 * max(1.0, np.abs(r).max()), name


def test_backward_matches_finite_differences():
    grid, D, k = (4, 4, 8), 8, 1
    inp, do, idx = inputs(grid, D, k, 32, H=1)
    scale = 0.4
    x = {n: oracle.bf16_to_f64(inp[n]) for n in "qkv"}

    def loss(xq, xk, xv):
        o, _ = oracle.forward(xq, xk, xv, grid, k, scale=scale, idx=idx)
        return float((o * do).sum())

    grads = dict(zip("qkv", oracle.backward(x["q"], x["k"], x["v"], do, grid, idx, scale)))
    rng = np.random.default_rng(5)
    h = 1e-6
    for name in "qkv":
        for _ in range(6):
            s, d = int(rng.integers(x[name].shape[1])), int(rng.integers(D))
            plus = {n: x[n].copy() for n in "qkv"}
            minus = {n: x[n].copy() for n in "qkv"}
            plus[name][0, s, 0, d] += h
            minus[name][0, s, 0, d] -= h
            fd = (loss(plus["q"], plus["k"], plus["v"]) - loss(minus["q"], minus["k"], minus["v"])) / (2 * h)
            assert abs(fd - grads[name][0, s, 0, d]) <= 1e-6 * max(1.0, abs(fd)), (name, s, d)


def test_constant_values_give_no_query_or_key_gradient():
    grid, D, k = (8, 8, 8), 16, 3
    inp, do, idx = inputs(grid, D, k, 33)
    v = np.zeros_like(inp["v"]) + workloads.round_to_bf16_bits(np.full(D, 0.75, dtype=np.float32))
    dq, dk, dv = oracle.backward(inp["q"], inp["k"], v, do, grid, idx)
    assert np.abs(dq).max() < 1e-12 and np.abs(dk).max() < 1e-12
    assert np.abs(dv).max() > 0.1


@pytest.mark.parametrize("grid", [(8, 8, 8), (5, 6, 7)])
def test_gradient_sums(grid):
    D, k = 16, 2
    inp, do, idx = inputs(grid, D, k, 34)
    dq, dk, dv = oracle.backward(inp["q"], inp["k"], inp["v"], do, grid, idx)
    # sum over key rows of dK is scale * sum_q (sum_keys dS) q = 0
    assert np.abs(dk.sum(axis=1)).max() < 1e-10
    # sum over key rows of dV is the sum of the output gradients (rows of P sum to 1)
    assert np.abs(dv.sum(axis=1) - do.sum(axis=1)).max() < 1e-10
