"""GPU parity: linear branch and combine (bf16(O_sparse + O_lin)) against the oracle,
both as two calls (vsa_sparse_attn_fwd with its fp32 output, then
vsa_linear_branch) and as the single fused pass (vsa_sparse_attn_linear_fwd).
The two-call chain is also run on raster Q with a raster output
(vsa_sparse_attn_fwd_raster with its fp32 cube-major output only, then
vsa_linear_branch with the RASTER layout): bit-identical to the cube-major
calls followed by the unpermute, in direct mode too; and the branch split
into vsa_linear_state and vsa_linear_apply is bit-identical to the one call.
The two run the same fp32 sums in the same order; where the compiler fuses
a multiply and an add in one kernel's combine but not in the other's, the
fp32 results differ in the last bits, and a few outputs land on the other
side of a bf16 rounding boundary.  Those last bits are relative to the two
operands O_sparse and O_lin, not to their sum, which can cancel: the two
outputs agree to two bf16 steps of the result plus 2^-20 (|O_sparse| +
|O_lin|), with at most one output in a thousand differing at all."""

import numpy as np
import pytest
import torch

import oracle
import workloads
from tests.gpu_util import assert_close, bf16_f64, to_dev

pytestmark = pytest.mark.gpu


def check_raster_chain(vsa, wl, inp, kc, vt, idx_d, of, out):
    """The layer's two-call chain on raster Q and output equals the cube-major calls bit for bit."""
    q = to_dev(inp["q"])
    of_r = torch.full_like(of, float("nan"))
    o_none, _ = vsa.sparse_attn_fwd_raster(q, kc, vt, idx_d, wl.grid, wl.softmax_scale, out_f32=of_r,
                                           bf16_out=False)
    assert o_none is None
    out_r = vsa.linear_branch(q, kc, vt, idx_d, of_r, wl.grid, raster=True)
    torch.cuda.synchronize()
    assert torch.equal(of_r, of), "raster fine stage: fp32 output differs"
    assert torch.equal(out_r, vsa.cube_unpermute(out, wl.grid)), "raster linear branch differs"
    # The branch in two parts (state pass, then the rest) on a fresh workspace.
    g = vsa.make_geom(wl.batch, wl.heads, wl.head_dim, wl.grid)
    ws = torch.full((vsa.workspace_bytes(g, linear=True),), 0xA5, dtype=torch.uint8, device="cuda:0")
    vsa.linear_state(kc, vt, wl.grid, ws)
    out_a = vsa.linear_apply(q, vt, idx_d, of, wl.grid, ws, raster=True)
    qc = vsa.cube_permute(q, wl.grid)
    out_c = vsa.linear_apply(qc, vt, idx_d, of, wl.grid, ws)
    torch.cuda.synchronize()
    assert torch.equal(out_a, out_r), "state + apply (raster) differs from the one call"
    assert torch.equal(out_c, out), "state + apply (token-major) differs from the one call"


def run(wl, inp, idx=None):
    import block_sparse_video_cube_amd as vsa

    valid = oracle.valid_rows(wl.grid)
    qc_o, kc_o, vc_o = (oracle.cube_permute(inp[n], wl.grid) for n in ("q", "k", "v"))
    if idx is None:
        idx = oracle.select_topk(qc_o, kc_o, valid, wl.topk)
    qc = vsa.cube_permute(to_dev(inp["q"]), wl.grid)
    kc = vsa.cube_permute(to_dev(inp["k"]), wl.grid)
    vt = vsa.cube_permute(to_dev(inp["v"]), wl.grid, layout="dim")
    idx_d = torch.from_numpy(np.ascontiguousarray(idx)).to("cuda:0")
    scale = wl.softmax_scale
    _, of, lse = vsa.sparse_attn_fwd(qc, kc, vt, idx_d, wl.grid, scale, want_f32=True, want_lse=True)
    out = vsa.linear_branch(qc, kc, vt, idx_d, of, wl.grid)
    fused, lse_f = vsa.sparse_attn_linear_fwd(qc, kc, vt, idx_d, wl.grid, scale, want_lse=True)
    check_raster_chain(vsa, wl, inp, kc, vt, idx_d, of, out)
    torch.cuda.synchronize()
    ref_s, _ = oracle.sparse_attention(qc_o, kc_o, vc_o, valid, idx, scale)
    ref_l = oracle.linear_branch(qc_o, kc_o, vc_o, valid, idx)
    ref = ref_s + ref_l
    a, f = bf16_f64(out), bf16_f64(fused)
    vt_ = torch.from_numpy(valid).to(lse.device)
    assert torch.equal(lse[:, :, vt_], lse_f[:, :, vt_]), "fused softmax branch: lse differs"
    d = np.abs(a - f)[:, :, valid]
    o_s = of.double().cpu().numpy()
    operands = (np.abs(o_s) + np.abs(a - o_s))[:, :, valid]
    step = 2.0 ** -7 * np.maximum(np.abs(a), np.abs(f))[:, :, valid] + 2.0 ** -20 * operands + 1e-30
    print(f"fused vs two calls: max |d| {d.max():.3e}, bound ratio {np.max(d / step):.2f}, "
          f"differing {np.count_nonzero(d)}/{d.size}")
    assert np.all(d <= 2 * step)
    assert np.count_nonzero(d) <= d.size // 1000 + 1
    assert_close(f[:, :, valid], ref[:, :, valid], "fused pass vs oracle")
    return a, ref, valid


CASES = [
    {"grid": (8, 8, 12), "topk": 2, "batch": 2, "heads": 2},
    {"grid": (8, 8, 12), "topk": 2, "head_dim": 64},
    {"grid": (5, 6, 7), "topk": 3, "heads": 2},             # ragged, padded keys excluded
    {"grid": (5, 6, 7), "topk": 3, "heads": 2, "head_dim": 64},
    {"grid": (16, 12, 16), "topk": 1, "heads": 1},          # 48 cubes, 47 unselected
    {"grid": (16, 12, 16), "topk": 10, "heads": 2, "batch": 2},
    # 728 query cubes, more than the fused pass's resident workgroups (one per
    # compute unit): each takes several cubes in turn, with the next cube's
    # first tiles loaded during the last steps of the one before; k = 11
    # also gives each cube a padded step.
    {"grid": (16, 28, 52), "topk": 11, "heads": 2, "batch": 1},
]


# More than half the cubes selected: the branch sums the unselected cubes
# directly (the total minus the selected part would magnify rounding).
DIRECT_CASES = [
    {"grid": (1, 9, 11), "topk": 8, "heads": 4, "head_dim": 64},   # one unselected cube of 16 or fewer keys
    {"grid": (5, 6, 7), "topk": 6, "heads": 2},
    {"grid": (16, 12, 16), "topk": 40, "heads": 2, "batch": 2},
    {"grid": (16, 12, 16), "topk": 47, "heads": 1, "head_dim": 64},
]


@pytest.mark.parametrize("over", DIRECT_CASES)
def test_hybrid_direct_sum_matches_oracle(over):
    import block_sparse_video_cube_amd as vsa

    wl = workloads.workload("hybrid").with_(**over)
    inp = workloads.make_inputs(wl)
    valid = oracle.valid_rows(wl.grid)
    qc_o, kc_o, vc_o = (oracle.cube_permute(inp[n], wl.grid) for n in ("q", "k", "v"))
    idx = oracle.select_topk(qc_o, kc_o, valid, wl.topk)
    ref = oracle.sparse_attention(qc_o, kc_o, vc_o, valid, idx, wl.softmax_scale)[0]
    ref = ref + oracle.linear_branch(qc_o, kc_o, vc_o, valid, idx)
    qc, kc = vsa.cube_permute(to_dev(inp["q"]), wl.grid), vsa.cube_permute(to_dev(inp["k"]), wl.grid)
    vt = vsa.cube_permute(to_dev(inp["v"]), wl.grid, layout="dim")
    idx_d = torch.from_numpy(idx).to("cuda:0")
    _, of, _ = vsa.sparse_attn_fwd(qc, kc, vt, idx_d, wl.grid, wl.softmax_scale, want_f32=True)
    out = vsa.linear_branch(qc, kc, vt, idx_d, of, wl.grid)
    check_raster_chain(vsa, wl, inp, kc, vt, idx_d, of, out)
    got = bf16_f64(out)
    assert_close(got[:, :, valid], ref[:, :, valid], f"hybrid direct {over}")
    with pytest.raises(vsa.VsaError):  # the fused pass takes at most half the cubes
        vsa.sparse_attn_linear_fwd(qc, kc, vt, idx_d, wl.grid, wl.softmax_scale)


@pytest.mark.parametrize("over", CASES)
def test_hybrid_matches_oracle(over):
    wl = workloads.workload("hybrid").with_(**over)
    inp = workloads.make_inputs(wl)
    got, ref, valid = run(wl, inp)
    assert_close(got[:, :, valid], ref[:, :, valid], f"hybrid {over}")


def test_all_cubes_selected_leaves_sparse_output():
    wl = workloads.workload("hybrid").with_(grid=(8, 8, 8), topk=8, batch=1, heads=2)
    inp = workloads.make_inputs(wl)
    got, ref, valid = run(wl, inp)
    assert_close(got[:, :, valid], ref[:, :, valid], "k = Nc")


def test_constant_values_give_twice_the_constant():
    # Both branches average V: with V = c everywhere the result is 2c.
    wl = workloads.workload("hybrid").with_(grid=(8, 8, 12), topk=2, batch=1, heads=2)
    inp = workloads.make_inputs(wl)
    inp["v"][:] = workloads.round_to_bf16_bits(np.full(inp["v"].shape, 0.75, np.float32))
    got, ref, valid = run(wl, inp)
    assert np.abs(got[:, :, valid] - 1.5).max() <= 1e-2
    assert np.abs(ref[:, :, valid] - 1.5).max() <= 1e-12
