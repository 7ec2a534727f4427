"""GPU parity of the linear branch's backward (vsa_linear_branch_bwd) against
the fp64 oracle (O11, pinned by torch autograd, finite differences and closed
forms), on the oracle's block lists.  Every case also runs the backward from
the forward's saved O_lin and 1/den (vsa_linear_branch with its o_lin and
inv_den outputs), which must give the recomputing pass's gradients bit for
bit.

Tolerance, against each gradient's own scale: max|d| <= 2^-6 max|ref| and
mean|d| <= 2^-7 mean|ref|.  Along each path the kernels round to bf16 (2^-9
relative) at six points in series: phi(Q) and phi(K); the forward's block
products phi(K) phi(Q)^T, which set O_lin and den; w = dO / den; the block
products W V^T and phi(Q) phi(K)^T before their second product; and the
output.  The totals S and M keep about 16 bits (bf16 hi + lo).  dQ and dK
are differences of two near-equal totals (S_U w against c z_U, M v against
m), so the same rounding weighs more there than in the softmax backward:
the same rounding points emulated in float64 on the first case below give
4.1e-3 (exact w) to 4.4e-3 (bf16 w) mean relative error for dQ, which is
what the kernels show, and 2^-7 = 7.8e-3 bounds it.
"""

import numpy as np
import pytest
import torch

import oracle
import workloads
from tests.gpu_util import assert_close_rel, bf16_f64, to_dev

pytestmark = pytest.mark.gpu

MAX_REL = 2.0 ** -6
MEAN_REL = 2.0 ** -7


def run(wl, seed, idx=None, heads=None):
    import block_sparse_video_cube_amd as vsa

    inp = workloads.make_inputs(wl)
    rng = np.random.default_rng(seed)
    do = workloads.round_to_bf16_bits(rng.standard_normal(inp["q"].shape).astype(np.float32))
    valid = oracle.valid_rows(wl.grid)
    qc_o, kc_o, vc_o, doc_o = (oracle.cube_permute(x, wl.grid) for x in (inp["q"], inp["k"], inp["v"], do))
    if idx is None:
        idx = oracle.select_topk(qc_o, kc_o, valid, wl.topk)
    q, k, v, dd = (to_dev(x) for x in (inp["q"], inp["k"], inp["v"], do))
    qc, kc, vc, doc = (vsa.cube_permute(x, wl.grid) for x in (q, k, v, dd))
    vt = vsa.cube_permute(v, wl.grid, layout="dim")
    idx_d = torch.from_numpy(np.ascontiguousarray(idx, dtype=np.int32)).to("cuda:0")
    got = vsa.linear_branch_bwd(qc, kc, vc, vt, idx_d, doc, wl.grid)
    # The same gradients from the forward's saved O_lin and 1/den.
    _, of, _ = vsa.sparse_attn_fwd(qc, kc, vt, idx_d, wl.grid, wl.softmax_scale, want_f32=True)
    _, saved = vsa.linear_branch(qc, kc, vt, idx_d, of, wl.grid, save=True)
    got_saved = vsa.linear_branch_bwd(qc, kc, vc, vt, idx_d, doc, wl.grid, saved=saved)
    torch.cuda.synchronize()
    for name, a, b in zip(("dq", "dk", "dv"), got, got_saved):
        assert torch.equal(a, b), f"{name}: saved-forward path differs from the recomputing one"
    print(f"[linear bwd {wl.grid} D={wl.head_dim} k={wl.topk}] oracle", flush=True)
    ref = oracle.linear_branch_bwd(qc_o, kc_o, vc_o, valid, idx, doc_o, heads=heads)
    return [bf16_f64(x) for x in got], ref, valid


CASES = [
    {"grid": (8, 8, 12), "topk": 2, "batch": 2, "heads": 2},
    {"grid": (8, 8, 12), "topk": 2, "head_dim": 64},
    {"grid": (5, 6, 7), "topk": 3, "heads": 2},             # ragged, padded keys and queries
    {"grid": (5, 6, 7), "topk": 3, "heads": 2, "head_dim": 64},
    {"grid": (16, 12, 16), "topk": 1, "heads": 1},          # 48 cubes, 47 unselected
    {"grid": (16, 12, 16), "topk": 10, "heads": 2, "batch": 2},
    # More than half the cubes selected: direct sums over the unselected cubes
    # (and, for dK and dV, over the query cubes that left a key cube out).
    {"grid": (1, 9, 11), "topk": 8, "heads": 2, "head_dim": 64},   # one unselected cube per row
    {"grid": (5, 6, 7), "topk": 6, "heads": 2},
    {"grid": (16, 12, 16), "topk": 40, "heads": 1, "batch": 2},
]


@pytest.mark.parametrize("over", CASES)
def test_linear_backward_matches_oracle(over):
    wl = workloads.workload("hybrid").with_(**over)
    got, ref, valid = run(wl, 300 + over["topk"])
    for name, g, r in zip(("dq", "dk", "dv"), got, ref):
        assert_close_rel(g[:, :, valid], r[:, :, valid], f"{name} {over}", MAX_REL, MEAN_REL)
        assert np.all(g[:, :, ~valid] == 0.0), f"{name}: padded rows"


def test_linear_backward_all_selected_is_zero():
    wl = workloads.workload("hybrid").with_(grid=(8, 8, 8), topk=8, batch=1, heads=2)
    got, ref, valid = run(wl, 310)
    for g in got:
        assert np.all(g == 0.0)


def test_linear_backward_hybrid_shape_one_head():
    # The hybrid layer's shape (364 cubes, k = 11, D = 128), one (b, h) checked.
    wl = workloads.workload("hybrid").with_(batch=1, heads=2)
    got, ref, valid = run(wl, 320, heads=[(0, 1)])
    for name, g, r in zip(("dq", "dk", "dv"), got, ref):
        assert_close_rel(g[0, 1][valid], r[0, 1][valid], f"{name} hybrid (0, 1)", MAX_REL, MEAN_REL)


def test_linear_backward_is_deterministic():
    # No atomics: two runs agree bit for bit (hybrid shape, one batch, two heads).
    import block_sparse_video_cube_amd as vsa

    wl = workloads.workload("hybrid").with_(batch=1, heads=2)
    inp = workloads.make_inputs(wl)
    rng = np.random.default_rng(330)
    do = workloads.round_to_bf16_bits(rng.standard_normal(inp["q"].shape).astype(np.float32))
    valid = oracle.valid_rows(wl.grid)
    idx = oracle.select_topk(oracle.cube_permute(inp["q"], wl.grid), oracle.cube_permute(inp["k"], wl.grid), valid,
                             wl.topk)
    q, k, v, dd = (to_dev(x) for x in (inp["q"], inp["k"], inp["v"], do))
    qc, kc, vc, doc = (vsa.cube_permute(x, wl.grid) for x in (q, k, v, dd))
    vt = vsa.cube_permute(v, wl.grid, layout="dim")
    idx_d = torch.from_numpy(np.ascontiguousarray(idx, dtype=np.int32)).to("cuda:0")
    first = vsa.linear_branch_bwd(qc, kc, vc, vt, idx_d, doc, wl.grid)
    again = vsa.linear_branch_bwd(qc, kc, vc, vt, idx_d, doc, wl.grid)
    torch.cuda.synchronize()
    for a, b in zip(first, again):
        assert torch.equal(a, b)
