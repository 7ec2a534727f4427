"""GPU parity at the largest cube count the library accepts (VSA_MAX_CUBES =
4096 cubes per head: a 64 x 64 x 64 latent grid), one head.

- top-k bit-exact on integer inputs (64 lane passes per row in the selection
  kernel), for a short and a long list;
- the bf16 fine stage, cube-major and raster, on sampled query cubes against
  the oracle (the oracle's lists fed in), raster bit-identical to cube-major;
- the fp8 stage on the same cubes against the oracle on the dequantized
  inputs, with the per-element bound of tests/test_gpu_fp8.py;
- the linear branch through summed states (D = 64 and 128) on sampled query
  cubes: their unselected sums and outputs against the oracle.
"""

import numpy as np
import pytest
import torch

import oracle
import workloads
from tests.gpu_util import assert_close, to_bits, to_dev
from tests.test_gpu_fp8 import check_vs_dequantized

pytestmark = pytest.mark.gpu

GRID = (64, 64, 64)


def wl_max(topk, D=64, seed=5000):
    return workloads.workload("tiny").with_(batch=1, heads=1, head_dim=D, grid=GRID, topk=topk, seed=seed)


@pytest.mark.parametrize("topk", [7, 410])
def test_topk_at_max_cubes_bit_exact(topk):
    import block_sparse_video_cube_amd as vsa

    wl = wl_max(topk)
    assert oracle.n_cubes(GRID) == 4096
    inp = workloads.make_integer_inputs(wl)
    qc = vsa.cube_permute(to_dev(inp["q"]), GRID)
    kc = vsa.cube_permute(to_dev(inp["k"]), GRID)
    got = vsa.select_topk(qc, kc, GRID, topk).cpu().numpy()
    print(f"[max cubes, k={topk}] oracle selection", flush=True)
    valid = oracle.valid_rows(GRID)
    ref = oracle.select_topk(oracle.cube_permute(inp["q"], GRID), oracle.cube_permute(inp["k"], GRID), valid, topk)
    assert np.array_equal(got, ref)


def test_fine_stage_at_max_cubes():
    import block_sparse_video_cube_amd as vsa

    wl = wl_max(64, D=128, seed=5100)
    inp = workloads.make_inputs(wl)
    valid = oracle.valid_rows(GRID)
    qc_o, kc_o, vc_o = (oracle.cube_permute(inp[n], GRID) for n in ("q", "k", "v"))
    idx = oracle.select_topk(qc_o, kc_o, valid, wl.topk)
    q, k, v = (to_dev(inp[n]) for n in ("q", "k", "v"))
    qc, kc = vsa.cube_permute(q, GRID), vsa.cube_permute(k, GRID)
    vt = vsa.cube_permute(v, GRID, layout="dim")
    idx_d = torch.from_numpy(np.ascontiguousarray(idx)).to("cuda:0")
    oc, _, _ = vsa.sparse_attn_fwd(qc, kc, vt, idx_d, GRID, wl.softmax_scale)
    o_r, _ = vsa.sparse_attn_fwd_raster(q, kc, vt, idx_d, GRID, wl.softmax_scale)
    assert torch.equal(o_r, vsa.cube_unpermute(oc, GRID))
    cubes = [0, 1, 63, 64, 1000, 2047, 2048, 3333, 4094, 4095]
    todo = [(0, 0, i) for i in cubes]
    print(f"[max cubes] oracle fine stage on {len(cubes)} cubes", flush=True)
    ref, _ = oracle.sparse_attention(qc_o, kc_o, vc_o, valid, idx, wl.softmax_scale, cubes=todo)
    rows = np.zeros(wl.rows, dtype=bool)
    for i in cubes:
        rows[64 * i:64 * i + 64] = True
    got = oracle.bf16_to_f64(to_bits(oc))
    assert_close(got[:, :, rows], ref[:, :, rows], "max cubes fine stage")


def test_fp8_stage_at_max_cubes():
    wl = wl_max(64, D=128, seed=5200)
    inp = workloads.make_inputs(wl)
    valid = oracle.valid_rows(GRID)
    idx = oracle.select_topk(oracle.cube_permute(inp["q"], GRID), oracle.cube_permute(inp["k"], GRID), valid,
                             wl.topk)
    cubes = [(0, 0, i) for i in (0, 511, 2048, 4095)]
    check_vs_dequantized(inp, GRID, idx, wl.softmax_scale, cubes, what="max cubes")


@pytest.mark.parametrize("D", [64, 128])
def test_linear_states_at_max_cubes(D):
    """The linear branch through summed states at 4096 cubes (64 state tiles per
    column, 32 ranges of 128 query cubes): sampled query cubes against the
    oracle (its lists fed in), the unselected sums of those cubes against the
    oracle's within the bf16 bound of tests/test_gpu_linear_states.py."""
    import block_sparse_video_cube_amd as vsa

    wl = wl_max(40, D=D, seed=5200 + D)
    inp = workloads.make_inputs(wl)
    valid = oracle.valid_rows(GRID)
    qc_o, kc_o, vc_o = (oracle.cube_permute(inp[n], GRID) for n in ("q", "k", "v"))
    idx = oracle.select_topk(qc_o, kc_o, valid, wl.topk)
    q, k, v = (to_dev(inp[n]) for n in ("q", "k", "v"))
    kc = vsa.cube_permute(k, GRID)
    vt = vsa.cube_permute(v, GRID, layout="dim")
    idx_d = torch.from_numpy(np.ascontiguousarray(idx)).to("cuda:0")
    st = vsa.linear_cube_states(kc, vt, GRID)
    su = vsa.linear_unselected(st, idx_d, GRID)
    o = vsa.sparse_attn_fwd_linear(q, kc, vt, idx_d, su, GRID, wl.softmax_scale)
    torch.cuda.synchronize()
    cubes = [0, 1, 127, 128, 1000, 2047, 2048, 3333, 4094, 4095]
    todo = [(0, 0, i) for i in cubes]
    print(f"[max cubes, D={D}] oracle sums and outputs on {len(cubes)} cubes", flush=True)
    S, z = oracle.linear_cube_states(kc_o, vc_o, valid)
    A, _ = oracle.linear_cube_states(kc_o, np.abs(oracle.bf16_to_f64(vc_o)), valid)
    u = 2.0 ** -8
    sug = su[0, 0, cubes].double().cpu().numpy()
    for c, row in zip(cubes, sug):
        keep = np.ones(4096, dtype=bool)
        keep[idx[0, 0, c]] = False
        s_ref, a_ref = S[0, 0, keep].sum(axis=0), A[0, 0, keep].sum(axis=0)
        bound = 1.02 * (u * (1 + u) * a_ref + u * np.abs(S[0, 0, keep]).sum(axis=0)) + u * np.abs(s_ref)
        got = row[:D * D].reshape(D, D).T  # stored [e][d]
        assert np.all(np.abs(got - s_ref) <= bound + 1e-30), c
        z_ref = z[0, 0, keep].sum(axis=0)
        assert np.all(np.abs(row[D * D:] - z_ref) <= (u * (2 + u) * 1.02 + u) * z_ref), c
    ref = oracle.sparse_attention(qc_o, kc_o, vc_o, valid, idx, wl.softmax_scale, cubes=todo)[0]
    ref = ref + oracle.linear_branch(qc_o, kc_o, vc_o, valid, idx, cubes=todo)
    rows = np.zeros(wl.rows, dtype=bool)
    for i in cubes:
        rows[64 * i:64 * i + 64] = True
    got = oracle.cube_permute(oracle.bf16_to_f64(to_bits(o)), GRID)
    assert_close(got[:, :, rows], ref[:, :, rows], f"max cubes linear states D={D}")
