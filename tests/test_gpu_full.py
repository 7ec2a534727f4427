"""GPU parity at the full workload sizes, on sampled outputs.

Each workload runs on the GPU through vsa.layer_forward, the function the
benchmark times, so the chain checked here is the benchmark's own: pooling of
Q, pooled permute of K, cube-transposed permute of V, selection from the
pooled means, and the raster-order fine stage (the hybrid layer: cube-major
rows, fine stage plus linear branch, unpermute; also the fused pass).  The
oracle then recomputes, for two sampled heads:
  - every block score row from the raster inputs: each GPU top-k row must be
    a valid top-k of the fp64 scores (near-tie band 1e-5 relative); rows
    identical to the oracle's are counted;
  - the output of sampled query cubes (first, last, partial and random ones)
    for the block lists the GPU chose (checked valid just before), compared
    at their raster token positions.
"""

import numpy as np
import pytest
import torch

import oracle
import workloads
from tests.gpu_util import assert_close, to_bits, to_dev, topk_valid_under

pytestmark = pytest.mark.gpu

SAMPLED_HEADS = {"wan1.3b": [0, 11], "wan14b": [3, 38], "720p": [0, 27], "hybrid": [5, 11], "sta": [2, 9]}


def sampled_cubes(wl, rng, n=20):
    valid = oracle.valid_rows(wl.grid).reshape(-1, 64)
    partial = [c for c in range(wl.n_cubes) if not valid[c].all()]
    cubes = {0, wl.n_cubes - 1}
    cubes.update(int(c) for c in rng.choice(wl.n_cubes, size=n, replace=False))
    if partial:
        cubes.update(int(c) for c in rng.choice(partial, size=min(8, len(partial)), replace=False))
    return sorted(cubes)


@pytest.mark.parametrize("name", ["wan1.3b", "wan14b", "720p", "hybrid", "sta"])
def test_full_size_sampled(name):
    import block_sparse_video_cube_amd as vsa

    wl = workloads.workload(name)
    heads = SAMPLED_HEADS[name]
    print(f"[{name}] generating inputs", flush=True)
    inp = workloads.make_inputs(wl)
    q, k, v = (to_dev(inp[n]) for n in ("q", "k", "v"))
    window = wl.window if wl.pattern == "sta" else None
    print(f"[{name}] GPU layer (the benchmark's chain)", flush=True)
    o, idx = vsa.layer_forward(q, k, v, wl.grid, wl.topk, wl.softmax_scale, linear=wl.linear, window=window)
    idx_gpu = idx.cpu().numpy()
    o_fused = None
    if wl.linear:
        o_fused, idx_f = vsa.layer_forward(q, k, v, wl.grid, wl.topk, wl.softmax_scale, linear=True,
                                           fused_linear=True)
        assert torch.equal(idx_f, idx)
    torch.cuda.synchronize()

    print(f"[{name}] oracle on heads {heads}", flush=True)
    sub = {n: np.ascontiguousarray(inp[n][:, :, heads, :]) for n in ("q", "k", "v")}
    valid = oracle.valid_rows(wl.grid)
    qc_o, kc_o, vc_o = (oracle.cube_permute(sub[n], wl.grid) for n in ("q", "k", "v"))
    idx_used = np.ascontiguousarray(idx_gpu[:, heads])
    if window is None:
        s = oracle.block_scores(oracle.cube_means(qc_o, valid), oracle.cube_means(kc_o, valid))
        ok = same = 0
        for b in range(wl.batch):
            for hi in range(len(heads)):
                for i in range(wl.n_cubes):
                    ok += topk_valid_under(s[b, hi, i], idx_used[b, hi, i], wl.topk)
                    same += np.array_equal(oracle.topk_row(s[b, hi, i], wl.topk), idx_used[b, hi, i])
        rows = wl.batch * len(heads) * wl.n_cubes
        print(f"[{name}] pooled top-k rows valid {ok}/{rows}, identical to the oracle {same}/{rows}")
        assert ok == rows
    else:
        ref_idx = oracle.sta_index(wl.grid, wl.window)
        assert all(np.array_equal(idx_used[b, hi], ref_idx) for b in range(wl.batch) for hi in range(len(heads)))

    rng = np.random.default_rng(7)
    cubes = sampled_cubes(wl, rng)
    todo = [(b, hi, i) for b in range(wl.batch) for hi in range(len(heads)) for i in cubes]
    ref, _ = oracle.sparse_attention(qc_o, kc_o, vc_o, valid, idx_used, wl.softmax_scale, cubes=todo)
    if wl.linear:
        ref = ref + oracle.linear_branch(qc_o, kc_o, vc_o, valid, idx_used, cubes=todo)
    rows_sel = np.zeros(wl.rows, dtype=bool)
    for i in cubes:
        rows_sel[64 * i:64 * i + 64] = True
    rows_sel &= valid
    # The sampled rows at their raster token positions.
    ref_tok = oracle.cube_unpermute(np.nan_to_num(ref, nan=0.0), wl.grid)
    tok_sel = oracle.cube_unpermute(np.broadcast_to(rows_sel[None, None, :, None], ref.shape[:3] + (1,)).copy(),
                                    wl.grid)[0, :, 0, 0]
    o_h = oracle.bf16_to_f64(to_bits(o[:, :, heads]))
    assert_close(o_h[:, tok_sel], ref_tok[:, tok_sel], f"[{name}] raster output ({len(cubes)} cubes per head)")
    if o_fused is not None:
        of_h = oracle.bf16_to_f64(to_bits(o_fused[:, :, heads]))
        assert_close(of_h[:, tok_sel], ref_tok[:, tok_sel], f"[{name}] fused pass, raster output")
