"""GPU parity: fine stage (block-sparse attention), fed the oracle's block lists.

Tolerance (bf16 output against the fp64 oracle, valid rows only): max-abs
2e-2 and mean-abs 2e-3.
"""

import math

import numpy as np
import pytest
import torch

import oracle
import workloads
from tests.gpu_util import assert_close, bf16_f64, to_dev

pytestmark = pytest.mark.gpu


def setup(wl, inp, idx=None):
    import block_sparse_video_cube_amd as vsa

    valid = oracle.valid_rows(wl.grid)
    qc_o, kc_o, vc_o = (oracle.cube_permute(inp[n], wl.grid) for n in ("q", "k", "v"))
    if idx is None:
        idx = oracle.select_topk(qc_o, kc_o, valid, wl.topk)
    qc = vsa.cube_permute(to_dev(inp["q"]), wl.grid)
    kc = vsa.cube_permute(to_dev(inp["k"]), wl.grid)
    vt = vsa.cube_permute(to_dev(inp["v"]), wl.grid, layout="dim")
    idx_d = torch.from_numpy(np.ascontiguousarray(idx)).to("cuda:0")
    return valid, (qc_o, kc_o, vc_o), idx, (qc, kc, vt, idx_d)


CASES = [
    # name, overrides
    ("tiny", {}),
    ("tiny", {"head_dim": 128}),
    ("tiny", {"grid": (5, 6, 7), "topk": 3, "heads": 3}),
    ("tiny", {"grid": (5, 6, 7), "topk": 3, "heads": 2, "head_dim": 128, "batch": 2}),
    ("tiny", {"grid": (9, 13, 6), "topk": 1}),
    ("tiny", {"grid": (12, 12, 12), "topk": 27, "head_dim": 128}),  # k = Nc: dense
    ("tiny", {"grid": (1, 1, 1), "topk": 1, "head_dim": 128}),        # one token
    ("wan1.3b", {"grid": (8, 12, 16), "topk": 5, "heads": 2}),        # per-head scales
    ("wan14b", {"grid": (8, 12, 16), "topk": 4, "heads": 2}),         # sinusoid
]


@pytest.mark.parametrize("name,over", CASES)
def test_fine_stage_matches_oracle(name, over):
    import block_sparse_video_cube_amd as vsa

    wl = workloads.workload(name).with_(**over)
    inp = workloads.make_inputs(wl)
    valid, (qc_o, kc_o, vc_o), idx, (qc, kc, vt, idx_d) = setup(wl, inp)
    scale = wl.softmax_scale
    oc, of, lse = vsa.sparse_attn_fwd(qc, kc, vt, idx_d, wl.grid, scale, want_f32=True, want_lse=True)
    torch.cuda.synchronize()
    ref, ref_lse = oracle.sparse_attention(qc_o, kc_o, vc_o, valid, idx, scale)
    assert_close(bf16_f64(oc)[:, :, valid], ref[:, :, valid], f"{name}{over} bf16")
    assert_close(of.cpu().numpy().astype(np.float64)[:, :, valid], ref[:, :, valid], f"{name}{over} f32",
                 max_abs=1e-2, mean_abs=1e-3)
    # The kernel's normaliser sums the bf16-rounded exponentials it applies to V
    # (unit roundoff 2^-8), so its lse is within ln(1 + 2^-8) = 3.9e-3 of the
    # exact value, plus fp32 noise.
    assert_close(lse.cpu().numpy().astype(np.float64)[:, :, valid], ref_lse[:, :, valid], f"{name}{over} lse",
                 max_abs=4.5e-3, mean_abs=1e-3)
    # Padded query rows hold finite values.
    assert torch.isfinite(oc.float()).all()


def test_fine_stage_constant_values_and_duplicates():
    import block_sparse_video_cube_amd as vsa

    wl = workloads.workload("tiny").with_(grid=(8, 8, 12), topk=3, head_dim=128)
    inp = workloads.make_inputs(wl)
    inp["v"][:] = workloads.round_to_bf16_bits(np.full(inp["v"].shape, -2.5, np.float32))
    idx = np.zeros((1, 2, wl.n_cubes, 3), dtype=np.int32)
    idx[..., 1] = 4
    idx[..., 2] = 4  # a duplicated block is simply counted twice
    valid, (qc_o, kc_o, vc_o), idx, (qc, kc, vt, idx_d) = setup(wl, inp, idx)
    oc, _, _ = vsa.sparse_attn_fwd(qc, kc, vt, idx_d, wl.grid, 0.1)
    assert np.all(bf16_f64(oc)[:, :, valid] == -2.5)


def test_fine_stage_is_deterministic():
    import block_sparse_video_cube_amd as vsa

    wl = workloads.workload("tiny").with_(grid=(8, 12, 16), topk=4, head_dim=128, heads=4)
    inp = workloads.make_inputs(wl)
    _, _, _, (qc, kc, vt, idx_d) = setup(wl, inp)
    first, _, _ = vsa.sparse_attn_fwd(qc, kc, vt, idx_d, wl.grid)
    for _ in range(10):
        again, _, _ = vsa.sparse_attn_fwd(qc, kc, vt, idx_d, wl.grid)
        assert torch.equal(first, again)


def test_large_logits_stay_finite():
    # Scores ~ 1e3 after scaling: the online softmax must not overflow.
    import block_sparse_video_cube_amd as vsa

    wl = workloads.workload("tiny").with_(grid=(8, 8, 8), topk=3, head_dim=64)
    inp = workloads.make_inputs(wl)
    big = workloads.bf16_bits_to_f32(inp["q"]) * 40.0
    inp["q"] = workloads.round_to_bf16_bits(big)
    valid, (qc_o, kc_o, vc_o), idx, (qc, kc, vt, idx_d) = setup(wl, inp)
    oc, _, _ = vsa.sparse_attn_fwd(qc, kc, vt, idx_d, wl.grid, 1.0)
    ref, _ = oracle.sparse_attention(qc_o, kc_o, vc_o, valid, idx, 1.0)
    assert_close(bf16_f64(oc)[:, :, valid], ref[:, :, valid], "large logits")
