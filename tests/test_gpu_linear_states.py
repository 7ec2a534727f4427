"""GPU parity: the linear branch through summed per-cube states
(vsa_linear_cube_states, vsa_linear_unselected, vsa_sparse_attn_fwd_linear)
against the oracle, step by step.

With u = 2^-8, the unit roundoff of bf16 rounding to nearest (8 significant
bits):
- The per-cube states (phi(K_j)^T V_j and the sums of phi(K_j), bf16) against
  the oracle's linear_cube_states: each value is an fp32 sum of products of
  the bf16-rounded phi(K) (relative error <= u) and V, rounded once to bf16,
  so its error is at most u (1 + u) A + u |S|, A the same sum over absolute
  values (phi(K) > 0, so A is the oracle's state of |V|).
- The unselected sums against the oracle's unselected_sums: fp32 sums of the
  bf16 states above, rounded once to bf16, so the bound is the state bound
  summed over the unselected cubes (times 1.02, which covers the (1 + u) of
  the final rounding and the fp32 sum) plus u |S_U|.
- The layer output (fine stage with the linear epilogue, fed the oracle's
  indices, raster Q and output) against oracle O_sparse + O_lin within the
  output tolerance, and against the tile chain (vsa_linear_branch) within a
  few bf16 steps.
"""

import numpy as np
import pytest
import torch

import oracle
import workloads
from tests.gpu_util import assert_close, bf16_f64, to_dev

pytestmark = pytest.mark.gpu


def run(wl, inp):
    import block_sparse_video_cube_amd as vsa

    B, H, D, nc = wl.batch, wl.heads, wl.head_dim, wl.n_cubes
    valid = oracle.valid_rows(wl.grid)
    qc_o, kc_o, vc_o = (oracle.cube_permute(inp[n], wl.grid) for n in ("q", "k", "v"))
    idx = oracle.select_topk(qc_o, kc_o, valid, wl.topk)
    q = to_dev(inp["q"])
    kc = vsa.cube_permute(to_dev(inp["k"]), wl.grid)
    vt = vsa.cube_permute(to_dev(inp["v"]), wl.grid, layout="dim")
    idx_d = torch.from_numpy(np.ascontiguousarray(idx)).to("cuda:0")
    # Poisoned outputs: every value must be written.
    st = vsa.linear_cube_states(kc, vt, wl.grid, out=torch.full((B, H, D + 1, nc, D), float("nan"),
                                                                dtype=torch.bfloat16, device="cuda:0"))
    su = vsa.linear_unselected(st, idx_d, wl.grid, out=torch.full((B, H, nc, D * D + D), float("nan"),
                                                                   dtype=torch.bfloat16, device="cuda:0"))
    out = vsa.sparse_attn_fwd_linear(q, kc, vt, idx_d, su, wl.grid, wl.softmax_scale, raster=True)
    qc = vsa.cube_permute(q, wl.grid)
    out_c = vsa.sparse_attn_fwd_linear(qc, kc, vt, idx_d, su, wl.grid, wl.softmax_scale, raster=False)
    _, of, _ = vsa.sparse_attn_fwd(qc, kc, vt, idx_d, wl.grid, wl.softmax_scale, want_f32=True)
    tiles = vsa.linear_branch(qc, kc, vt, idx_d, of, wl.grid)
    torch.cuda.synchronize()

    # Step 1: per-cube states.
    S_o, z_o = oracle.linear_cube_states(kc_o, vc_o, valid)
    A_o, za_o = oracle.linear_cube_states(kc_o, np.abs(oracle.bf16_to_f64(vc_o)), valid)
    stg = st.double().cpu().numpy()                      # [B, H, D + 1, nc, D]: [e][j][d]
    S_g = np.transpose(stg[:, :, :D], (0, 1, 3, 4, 2))   # -> [B, H, nc, d, e]
    z_g = stg[:, :, D]                                   # [B, H, nc, d]
    u = 2.0 ** -8
    bound_s = u * (1 + u) * A_o + u * np.abs(S_o) + 1e-30
    bound_z = u * (1 + u) * za_o + u * np.abs(z_o) + 1e-30
    assert np.all(np.isfinite(S_g)) and np.all(np.isfinite(z_g))
    print(f"states: max err/bound {np.max(np.abs(S_g - S_o) / bound_s):.3f}, "
          f"z {np.max(np.abs(z_g - z_o) / bound_z):.3f}")
    assert np.all(np.abs(S_g - S_o) <= bound_s) and np.all(np.abs(z_g - z_o) <= bound_z)

    # Step 2: sums over the unselected cubes.
    Su_o, zu_o = oracle.unselected_sums(S_o, z_o, idx)
    Au_o, zau_o = oracle.unselected_sums(bound_s, bound_z, idx)
    sug = su.double().cpu().numpy()
    Su_g = np.transpose(sug[..., :D * D].reshape(B, H, nc, D, D), (0, 1, 2, 4, 3))  # stored [e][d]
    zu_g = sug[..., D * D:]
    # (1.02: the rounding of the fp32 sum also scales the summed state errors,
    # and the fp32 sum of up to a few thousand terms adds far less than 1 %.)
    bsu = 1.02 * Au_o + u * np.abs(Su_o) + 1e-30
    bzu = 1.02 * zau_o + u * np.abs(zu_o) + 1e-30
    assert np.all(np.isfinite(Su_g)) and np.all(np.isfinite(zu_g))
    print(f"unselected sums: max err/bound {np.max(np.abs(Su_g - Su_o) / bsu):.3f}, "
          f"z {np.max(np.abs(zu_g - zu_o) / bzu):.3f}")
    assert np.all(np.abs(Su_g - Su_o) <= bsu) and np.all(np.abs(zu_g - zu_o) <= bzu)

    # Step 3: the layer output.
    ref = oracle.sparse_attention(qc_o, kc_o, vc_o, valid, idx, wl.softmax_scale)[0]
    ref = ref + oracle.linear_branch(qc_o, kc_o, vc_o, valid, idx)
    got_c = bf16_f64(out_c)
    assert torch.equal(vsa.cube_unpermute(out_c, wl.grid), out), "raster and cube-major outputs differ"
    t = bf16_f64(tiles)
    d = np.abs(got_c - t)[:, :, valid]
    print(f"states vs tiles: max |d| {d.max():.3e}, differing {np.count_nonzero(d)}/{d.size}")
    assert np.all(d <= 2.0 ** -6 * np.maximum(np.abs(got_c), np.abs(t))[:, :, valid] + 1e-3)
    return got_c, ref, valid


CASES = [
    {"grid": (8, 8, 12), "topk": 2, "batch": 2, "heads": 2},
    {"grid": (8, 8, 12), "topk": 2, "head_dim": 64},
    {"grid": (5, 6, 7), "topk": 3, "heads": 2},             # ragged: padded keys excluded, padded queries dropped
    {"grid": (9, 5, 6), "topk": 4, "heads": 2, "head_dim": 64},
    {"grid": (16, 12, 16), "topk": 1, "heads": 1},          # 48 cubes, 47 unselected
    {"grid": (16, 12, 16), "topk": 40, "heads": 2},         # most cubes selected
    # 364 cubes: three ranges of 128 query cubes and six 64-cube state tiles,
    # the last one partial.
    {"grid": (16, 28, 52), "topk": 11, "heads": 1, "batch": 1},
    {"grid": (13, 10, 22), "topk": 5, "heads": 2, "batch": 1},
]


@pytest.mark.parametrize("over", CASES)
def test_states_path_matches_oracle(over):
    wl = workloads.workload("hybrid").with_(**over)
    inp = workloads.make_inputs(wl)
    got, ref, valid = run(wl, inp)
    assert_close(got[:, :, valid], ref[:, :, valid], f"hybrid (states) {over}")


def test_states_path_all_selected_leaves_sparse_output():
    import block_sparse_video_cube_amd as vsa

    wl = workloads.workload("hybrid").with_(grid=(8, 8, 8), topk=8, batch=1, heads=2)
    inp = workloads.make_inputs(wl)
    got, ref, valid = run(wl, inp)
    assert_close(got[:, :, valid], ref[:, :, valid], "k = Nc")
    # Nothing unselected: the output is the fine stage's alone (the epilogue
    # adds an exact zero; its fp32 combine may contract differently, so up to
    # one bf16 step).
    q = to_dev(inp["q"])
    kc = vsa.cube_permute(to_dev(inp["k"]), wl.grid)
    vt = vsa.cube_permute(to_dev(inp["v"]), wl.grid, layout="dim")
    idx = torch.arange(wl.n_cubes, dtype=torch.int32, device="cuda:0").repeat(1, 2, wl.n_cubes, 1)
    su = vsa.linear_unselected(vsa.linear_cube_states(kc, vt, wl.grid), idx, wl.grid)
    out = vsa.sparse_attn_fwd_linear(q, kc, vt, idx, su, wl.grid, wl.softmax_scale)
    alone, _ = vsa.sparse_attn_fwd_raster(q, kc, vt, idx, wl.grid, wl.softmax_scale)
    torch.cuda.synchronize()
    assert not su.any()
    a, b = bf16_f64(out), bf16_f64(alone)
    assert np.all(np.abs(a - b) <= 2.0 ** -8 * np.abs(b) + 1e-30)


def test_states_path_constant_values_give_twice_the_constant():
    # Both branches average V: with V = c everywhere the result is 2c.
    wl = workloads.workload("hybrid").with_(grid=(8, 8, 12), topk=2, batch=1, heads=2)
    inp = workloads.make_inputs(wl)
    inp["v"][:] = workloads.round_to_bf16_bits(np.full(inp["v"].shape, 0.75, np.float32))
    got, ref, valid = run(wl, inp)
    assert np.abs(got[:, :, valid] - 1.5).max() <= 1e-2
    assert np.abs(ref[:, :, valid] - 1.5).max() <= 1e-12


def test_layer_forward_states_matches_oracle():
    """The hybrid layer as the benchmark runs it (linear_mode="states"): its own
    selection (checked a valid top-k of the oracle's fp64 scores) and the output
    for that selection against the oracle."""
    import block_sparse_video_cube_amd as vsa
    from tests.gpu_util import topk_valid_under

    wl = workloads.workload("hybrid").with_(grid=(13, 10, 22), topk=5, batch=2, heads=2)
    inp = workloads.make_inputs(wl)
    out, idx = vsa.layer_forward(to_dev(inp["q"]), to_dev(inp["k"]), to_dev(inp["v"]), wl.grid, wl.topk,
                                 wl.softmax_scale, linear=True)
    torch.cuda.synchronize()
    idx = idx.cpu().numpy()
    valid = oracle.valid_rows(wl.grid)
    qc_o, kc_o, vc_o = (oracle.cube_permute(inp[n], wl.grid) for n in ("q", "k", "v"))
    sc = oracle.block_scores(oracle.cube_means(qc_o, valid), oracle.cube_means(kc_o, valid))
    for b in range(wl.batch):
        for h in range(wl.heads):
            for i in range(wl.n_cubes):
                assert topk_valid_under(sc[b, h, i], idx[b, h, i], wl.topk), (b, h, i)
    ref = oracle.sparse_attention(qc_o, kc_o, vc_o, valid, idx, wl.softmax_scale)[0]
    ref = ref + oracle.linear_branch(qc_o, kc_o, vc_o, valid, idx)
    got = oracle.cube_permute(oracle.bf16_to_f64(np.ascontiguousarray(
        out.cpu().view(torch.int16).numpy().view(np.uint16))), wl.grid)
    assert_close(got[:, :, valid], ref[:, :, valid], "layer_forward (states)")
