"""Property test of the whole layer on the GPU against the oracle (Hypothesis).

Random small layers: latent grid T, H, W in 1..12 (non-multiples of 4 give
partial cubes, and so the packed fine stage), D in {64, 128}, k in [1, Nc],
B * heads <= 4, with and without the linear branch.  Each runs through
vsa.layer_forward, the benchmark's chain.  Checked per example:
  - every top-k row is a valid top-k of the oracle's fp64 block scores
    (near-tie band 1e-5 relative);
  - the raster output equals the oracle's (fine stage, plus the linear
    branch) for the lists the GPU chose, within 2e-2 max-abs / 2e-3
    mean-abs;
  - with the linear branch and k <= Nc / 2 or k = Nc, the single fused pass
    (vsa_sparse_attn_linear_fwd) chooses the same lists and meets the same
    bound.
Examples are derandomized (the same cases every run), bounded in number, and
the run stops at the first failure (no shrinking on the GPU).
"""

import numpy as np
import pytest
from hypothesis import HealthCheck, Phase, given, settings
from hypothesis import strategies as st

import oracle
import workloads
from tests.gpu_util import assert_close, bf16_f64, to_dev, topk_valid_under

pytestmark = pytest.mark.gpu


@st.composite
def layers(draw):
    grid = tuple(draw(st.integers(1, 12)) for _ in range(3))
    nc = oracle.n_cubes(grid)
    batch = draw(st.integers(1, 2))
    heads = draw(st.integers(1, 4 // batch))
    return dict(grid=grid, D=draw(st.sampled_from([64, 128])), topk=draw(st.integers(1, nc)),
                batch=batch, heads=heads, linear=draw(st.booleans()), seed=draw(st.integers(0, 10_000)))


def check_layer(grid, D, topk, batch, heads, linear, seed):
    import torch

    import block_sparse_video_cube_amd as vsa

    wl = workloads.workload("tiny").with_(grid=grid, head_dim=D, topk=topk, batch=batch, heads=heads,
                                          seed=2000 + seed, linear=linear)
    inp = workloads.make_inputs(wl)
    o, idx = vsa.layer_forward(to_dev(inp["q"]), to_dev(inp["k"]), to_dev(inp["v"]), grid, topk,
                               wl.softmax_scale, linear=linear)
    torch.cuda.synchronize()
    idx = idx.cpu().numpy()
    valid = oracle.valid_rows(grid)
    qc, kc, vc = (oracle.cube_permute(inp[n], grid) for n in ("q", "k", "v"))
    s = oracle.block_scores(oracle.cube_means(qc, valid), oracle.cube_means(kc, valid))
    for b in range(batch):
        for h in range(heads):
            for i in range(wl.n_cubes):
                assert topk_valid_under(s[b, h, i], idx[b, h, i], topk), (b, h, i)
    ref, _ = oracle.sparse_attention(qc, kc, vc, valid, idx, wl.softmax_scale)
    if linear:
        ref = ref + oracle.linear_branch(qc, kc, vc, valid, idx)
    ref_tok = oracle.cube_unpermute(np.nan_to_num(ref), grid)
    assert_close(bf16_f64(o), ref_tok, f"layer {grid} D={D} k={topk} B={batch} heads={heads} linear={linear}")
    if linear and (2 * topk <= wl.n_cubes or topk == wl.n_cubes):
        o_f, idx_f = vsa.layer_forward(to_dev(inp["q"]), to_dev(inp["k"]), to_dev(inp["v"]), grid, topk,
                                       wl.softmax_scale, linear=True, fused_linear=True)
        torch.cuda.synchronize()
        assert np.array_equal(idx_f.cpu().numpy(), idx)
        assert_close(bf16_f64(o_f), ref_tok, f"fused layer {grid} D={D} k={topk} B={batch} heads={heads}")


@settings(max_examples=40, deadline=None, derandomize=True, database=None,
          phases=[Phase.explicit, Phase.generate], suppress_health_check=list(HealthCheck))
@given(layers())
def test_layer_matches_oracle(case):
    print(case, flush=True)
    check_layer(**case)
