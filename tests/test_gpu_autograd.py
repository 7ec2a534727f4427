"""The layer as a torch autograd node (vsa_attention with inputs that require
gradients): its backward runs the library's kernels (the fine stage's, plus
the linear branch's with the fine stage's gradients as addends), compared with
the fp64 oracle's gradients (O9, O9 + O11 for the hybrid layer).

Tolerances as for the kernels alone: each gradient within 2^-6 (max) of its
own scale, and 2^-8 (mean) for the fine stage, 2^-7 (mean) with the linear
branch (one bf16 rounding of the sum)."""

import numpy as np
import pytest
import torch

import oracle
import workloads
from tests.gpu_util import assert_close_rel, bf16_f64, to_dev

pytestmark = pytest.mark.gpu

CASES = [
    ("sparse", {"grid": (8, 8, 12), "topk": 3, "heads": 2}, False, 2.0 ** -8),
    ("sparse-ragged", {"grid": (5, 6, 7), "topk": 3, "heads": 2, "head_dim": 64}, False, 2.0 ** -8),
    ("hybrid", {"grid": (8, 8, 12), "topk": 2, "batch": 2, "heads": 2}, True, 2.0 ** -7),
    ("hybrid-ragged", {"grid": (5, 6, 7), "topk": 3, "heads": 2}, True, 2.0 ** -7),
]


@pytest.mark.parametrize("name,over,linear,mean_rel", CASES)
def test_autograd_matches_oracle(name, over, linear, mean_rel):
    import block_sparse_video_cube_amd as vsa

    wl = workloads.workload("hybrid" if linear else "tiny").with_(**over)
    inp = workloads.make_inputs(wl)
    rng = np.random.default_rng(900 + wl.topk)
    do = workloads.round_to_bf16_bits(rng.standard_normal(inp["q"].shape).astype(np.float32))
    q, k, v = (to_dev(inp[n]).requires_grad_(True) for n in ("q", "k", "v"))
    o, idx = vsa.vsa_attention(q, k, v, wl.grid, wl.topk, wl.softmax_scale, linear=linear)
    o.backward(to_dev(do))
    torch.cuda.synchronize()
    idx_np = idx.cpu().numpy()
    print(f"[autograd {name}] oracle", flush=True)
    ref = list(oracle.backward(inp["q"], inp["k"], inp["v"], oracle.bf16_to_f64(do), wl.grid, idx_np,
                               wl.softmax_scale))
    if linear:
        valid = oracle.valid_rows(wl.grid)
        cm = [oracle.cube_permute(x, wl.grid) for x in (inp["q"], inp["k"], inp["v"], do)]
        lin = oracle.linear_branch_bwd(*cm[:3], valid, idx_np, oracle.bf16_to_f64(cm[3]))
        ref = [r + oracle.cube_unpermute(x, wl.grid) for r, x in zip(ref, lin)]
    for gname, t, r in zip(("dq", "dk", "dv"), (q, k, v), ref):
        assert_close_rel(bf16_f64(t.grad), r, f"{gname} {name}", 2.0 ** -6, mean_rel)
