"""Pins of the oracle's linear-branch backward (O11), independent of its code.

- torch autograd (CPU, float64) through a dense token-level form of O6:
  O_lin = ((phi(Q) phi(K)^T) * M) V / rowsum((phi(Q) phi(K)^T) * M), with
  M[q, r] = 1 where key row r is valid and its cube is not selected by q's
  cube, and phi = elu + 1 from torch: a library's chain rule and feature map,
  not the oracle's formulas;
- central finite differences of sum(O_lin * dO) through the oracle's forward;
- closed forms: V constant gives dQ = dK = 0; the dV rows of a head sum to the
  sum of the dO rows of query cubes with unselected cubes (each output row is
  an average of value rows with weights summing to 1); with every cube
  selected there is no gradient.
"""

import numpy as np
import pytest
import torch

import oracle
import workloads

CASES = [
    # (grid, D, k)
    ((8, 8, 8), 16, 2),
    ((5, 6, 7), 8, 3),     # partial cubes: padded keys and queries
    ((4, 8, 12), 16, 5),   # 6 cubes, one left unselected per row
]


def setup(grid, D, k, seed, H=2, const_v=None):
    wl = workloads.workload("tiny").with_(heads=H, head_dim=D, grid=grid, topk=k, seed=seed)
    inp = workloads.make_inputs(wl)
    valid = oracle.valid_rows(grid)
    qc, kc, vc = (oracle.bf16_to_f64(oracle.cube_permute(inp[n], grid)) for n in "qkv")
    if const_v is not None:
        vc = np.where(valid[None, None, :, None], const_v, 0.0) * np.ones_like(vc)
    idx = oracle.select_topk(oracle.cube_permute(inp["q"], grid), oracle.cube_permute(inp["k"], grid), valid, k)
    rng = np.random.default_rng(seed + 7)
    doc = rng.standard_normal(qc.shape) * valid[None, None, :, None]
    return qc, kc, vc, valid, idx, doc


def torch_dense_grads(qc, kc, vc, valid, idx, doc):
    B, H, Np, D = qc.shape
    cube = np.arange(Np) // 64
    grads = [np.zeros_like(qc) for _ in range(3)]
    for b in range(B):
        for h in range(H):
            m = np.zeros((Np, Np))
            for r in range(Np):
                m[r] = valid & ~np.isin(cube, idx[b, h, cube[r]])
            mask = torch.from_numpy(m)
            tq, tk, tv = (torch.tensor(x[b, h], requires_grad=True) for x in (qc, kc, vc))
            fq = torch.nn.functional.elu(tq) + 1.0
            fk = torch.nn.functional.elu(tk) + 1.0
            a = (fq @ fk.T) * mask
            den = a.sum(dim=1, keepdim=True)
            has = den > 0
            o = torch.where(has, (a @ tv) / torch.where(has, den, torch.ones_like(den)), torch.zeros_like(den))
            (o * torch.from_numpy(doc[b, h] * valid[:, None])).sum().backward()
            for g, t in zip(grads, (tq, tk, tv)):
                g[b, h] = t.grad.numpy() * valid[:, None]
    return grads


@pytest.mark.parametrize("grid,D,k", CASES)
def test_linear_backward_matches_torch_autograd(grid, D, k):
    qc, kc, vc, valid, idx, doc = setup(grid, D, k, 40 + D)
    got = oracle.linear_branch_bwd(qc, kc, vc, valid, idx, doc)
    ref = torch_dense_grads(qc, kc, vc, valid, idx, doc)
    for name, g, r in zip("qkv", got, ref):
        assert np.allclose(g, r, rtol=1e-10, atol=1e-12), name


def test_linear_backward_matches_finite_differences():
    grid, D, k = (4, 8, 8), 4, 1
    qc, kc, vc, valid, idx, doc = setup(grid, D, k, 61, H=1)

    def loss(xq, xk, xv):
        return float((oracle.linear_branch(xq, xk, xv, valid, idx) * doc).sum())

    x = {"q": qc, "k": kc, "v": vc}
    grads = dict(zip("qkv", oracle.linear_branch_bwd(qc, kc, vc, valid, idx, doc)))
    rng = np.random.default_rng(9)
    h = 1e-6
    for name in "qkv":
        for _ in range(8):
            r, d = int(rng.integers(qc.shape[2])), int(rng.integers(D))
            plus = {n: x[n].copy() for n in "qkv"}
            minus = {n: x[n].copy() for n in "qkv"}
            plus[name][0, 0, r, d] += h
            minus[name][0, 0, r, d] -= h
            fd = (loss(plus["q"], plus["k"], plus["v"]) - loss(minus["q"], minus["k"], minus["v"])) / (2 * h)
            assert abs(fd - grads[name][0, 0, r, d]) <= 1e-6 * max(1.0, abs(fd)), (name, r, d)


def test_constant_values_give_no_query_or_key_gradient():
    qc, kc, vc, valid, idx, doc = setup((8, 8, 8), 16, 2, 77, const_v=0.75)
    dq, dk, dv = oracle.linear_branch_bwd(qc, kc, vc, valid, idx, doc)
    assert np.abs(dq).max() < 1e-12 and np.abs(dk).max() < 1e-12
    # Every query cube has unselected cubes (k = 2 of 8): dV rows sum to the dO rows' sum.
    assert np.allclose(dv.sum(axis=2), doc.sum(axis=2), rtol=1e-10, atol=1e-10)


def test_all_cubes_selected_gives_no_gradient():
    qc, kc, vc, valid, idx, doc = setup((8, 8, 8), 16, 8, 78)
    for g in oracle.linear_branch_bwd(qc, kc, vc, valid, idx, doc):
        assert np.all(g == 0.0)
