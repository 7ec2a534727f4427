"""GPU parity of the fine-stage backward (dQ, dK, dV) against the fp64 oracle.

The GPU runs the forward (for O and lse) and the backward through the C ABI
on the oracle's block lists; the oracle differentiates the same attention in
fp64 (its own pins: torch autograd, finite differences, closed forms).

Tolerance, measured against each gradient's own scale:
max|d| <= 2^-6 max|ref| and mean|d| <= 2^-8 mean|ref|.  Derivation: the
backward recovers P = exp(scale S - lse) from the forward's lse, which is the
log of the sum of the bf16-rounded weights, so every weight carries a
systematic relative error of at most 2^-8; the matrix-core operands P and dS
and the forward output O used in rowsum(dO * O) are bf16 (2^-9 relative each),
and the outputs are rounded once to bf16 (2^-9).  The sum, 2^-7, taken
against the largest entry of the tensor, is doubled for the max bound; the
mean error stays near the 2^-8 systematic term.
"""

import numpy as np
import pytest
import torch

import oracle
import workloads
from tests.gpu_util import assert_close_rel, to_bits, to_dev

pytestmark = pytest.mark.gpu

MAX_REL = 2.0 ** -6
MEAN_REL = 2.0 ** -8


def grad_out(shape, seed):
    rng = np.random.default_rng(seed)
    return workloads.round_to_bf16_bits(rng.standard_normal(shape).astype(np.float32))


def gpu_backward(inp, do_bits, grid, idx_np, scale):
    import block_sparse_video_cube_amd as vsa

    q, k, v, do = (to_dev(x) for x in (inp["q"], inp["k"], inp["v"], do_bits))
    qc, kc, vc, doc = (vsa.cube_permute(x, grid) for x in (q, k, v, do))
    vt = vsa.cube_permute(v, grid, layout="dim")
    idx = torch.from_numpy(np.ascontiguousarray(idx_np, dtype=np.int32)).to("cuda:0")
    oc, _, lse = vsa.sparse_attn_fwd(qc, kc, vt, idx, grid, scale, want_lse=True)
    dq, dk, dv = vsa.sparse_attn_bwd(qc, kc, vc, oc, doc, lse, idx, grid, scale)
    out = tuple(vsa.cube_unpermute(x, grid) for x in (dq, dk, dv))
    torch.cuda.synchronize()
    return tuple(oracle.bf16_to_f64(to_bits(x)) for x in out)


CASES = [
    # (name, B, H, D, grid, k)
    ("tiny", 1, 2, 64, (8, 8, 8), 2),
    ("d128", 1, 2, 128, (8, 12, 16), 5),
    ("partial", 2, 1, 128, (9, 14, 13), 4),
    ("partial64", 1, 3, 64, (5, 6, 7), 3),
    ("dense", 1, 1, 128, (8, 8, 12), 12),
    ("k1", 1, 2, 64, (8, 8, 8), 1),
]


@pytest.mark.parametrize("name,B,H,D,grid,k", CASES)
def test_backward_matches_oracle(name, B, H, D, grid, k):
    wl = workloads.workload("tiny").with_(batch=B, heads=H, head_dim=D, grid=grid, topk=k, seed=2000 + len(name))
    inp = workloads.make_inputs(wl)
    do = grad_out(inp["q"].shape, 77 + k)
    valid = oracle.valid_rows(grid)
    idx = oracle.select_topk(oracle.cube_permute(inp["q"], grid), oracle.cube_permute(inp["k"], grid), valid, k)
    got = gpu_backward(inp, do, grid, idx, wl.softmax_scale)
    ref = oracle.backward(inp["q"], inp["k"], inp["v"], do, grid, idx, wl.softmax_scale)
    for what, g_, r in zip(("dq", "dk", "dv"), got, ref):
        assert_close_rel(g_, r, f"{name} {what}", MAX_REL, MEAN_REL)


def test_backward_unselected_key_cube_gets_zero():
    # Every query cube selects only cube 0 and its own cube: other key cubes get no gradient.
    grid, D = (8, 8, 8), 64
    wl = workloads.workload("tiny").with_(heads=1, head_dim=D, grid=grid, topk=2, seed=2100)
    inp = workloads.make_inputs(wl)
    do = grad_out(inp["q"].shape, 78)
    nc = oracle.n_cubes(grid)
    idx = np.array([[sorted({0, i} | ({1} if i == 0 else set())) for i in range(nc)]], dtype=np.int32)[None]
    got = gpu_backward(inp, do, grid, idx, wl.softmax_scale)
    ref = oracle.backward(inp["q"], inp["k"], inp["v"], do, grid, idx, wl.softmax_scale)
    for what, g_, r in zip(("dq", "dk", "dv"), got, ref):
        assert_close_rel(g_, r, f"own+first {what}", MAX_REL, MEAN_REL)


@pytest.mark.parametrize("name,heads", [("wan1.3b", [0]), ("720p", [5])])
def test_backward_full_size_sampled_heads(name, heads):
    wl = workloads.workload(name)
    full = workloads.make_inputs(wl, heads=heads)
    sub = {n: np.ascontiguousarray(full[n][:, :, heads, :]) for n in ("q", "k", "v")}
    del full
    do = grad_out(sub["q"].shape, 79)
    valid = oracle.valid_rows(wl.grid)
    idx = oracle.select_topk(oracle.cube_permute(sub["q"], wl.grid), oracle.cube_permute(sub["k"], wl.grid),
                             valid, wl.topk)
    print(f"[{name}] GPU backward on {len(heads)} head(s)", flush=True)
    got = gpu_backward(sub, do, wl.grid, idx, wl.softmax_scale)
    print(f"[{name}] oracle backward", flush=True)
    ref = oracle.backward(sub["q"], sub["k"], sub["v"], do, wl.grid, idx, wl.softmax_scale)
    for what, g_, r in zip(("dq", "dk", "dv"), got, ref):
        assert_close_rel(g_, r, f"{name} {what}", MAX_REL, MEAN_REL)


def test_backward_is_deterministic():
    # No atomics: two runs (the second with a fresh workspace) agree bit for bit,
    # at the Wan2.1-1.3B shape with two heads.
    import block_sparse_video_cube_amd as vsa

    wl = workloads.workload("wan1.3b").with_(heads=2)
    inp = workloads.make_inputs(wl)
    do = grad_out(inp["q"].shape, 4242)
    valid = oracle.valid_rows(wl.grid)
    idx = oracle.select_topk(oracle.cube_permute(inp["q"], wl.grid), oracle.cube_permute(inp["k"], wl.grid), valid,
                             wl.topk)
    q, k, v, dd = (to_dev(x) for x in (inp["q"], inp["k"], inp["v"], do))
    qc, kc, vc, doc = (vsa.cube_permute(x, wl.grid) for x in (q, k, v, dd))
    vt = vsa.cube_permute(v, wl.grid, layout="dim")
    idx_d = torch.from_numpy(np.ascontiguousarray(idx, dtype=np.int32)).to("cuda:0")
    oc, _, lse = vsa.sparse_attn_fwd(qc, kc, vt, idx_d, wl.grid, wl.softmax_scale, want_lse=True)
    first = vsa.sparse_attn_bwd(qc, kc, vc, oc, doc, lse, idx_d, wl.grid, wl.softmax_scale)
    again = vsa.sparse_attn_bwd(qc, kc, vc, oc, doc, lse, idx_d, wl.grid, wl.softmax_scale)
    torch.cuda.synchronize()
    for a, b in zip(first, again):
        assert torch.equal(a, b)
