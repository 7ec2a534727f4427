"""The allocation-free quantizer entry point (vsa_quant_fp8_noalloc) against
vsa_quant_fp8 with a caller workspace: the same kernels, so every output must
match bit for bit.  Two calls in a row on one device, the second on a smaller
problem, so the second must clear what the first left in the static scratch.
Called through the C ABI (ctypes) with preallocated outputs."""

import ctypes

import numpy as np
import pytest
import torch

import workloads
from tests.gpu_util import to_dev

pytestmark = pytest.mark.gpu


def outputs(B, H, D, nc, rows, means):
    u8 = dict(dtype=torch.uint8, device="cuda:0")
    f32 = dict(dtype=torch.float32, device="cuda:0")
    return [torch.full((B, H, rows, D), 7, **u8), torch.full((B, H, nc), -1.0, **f32),
            torch.full((B, H, rows, D), 7, **u8), torch.full((B, H, nc), -1.0, **f32),
            torch.full((B, H, nc, D, 64), 7, **u8), torch.full((B, H, D), -1.0, **f32),
            torch.full((B, H, nc, D), -1.0, **f32) if means else None,
            torch.full((B, H, nc, D), -1.0, **f32) if means else None]


def ptr(t):
    return t.data_ptr() if t is not None else None


@pytest.mark.parametrize("order", ["large_then_small"])
def test_noalloc_quant_matches_workspace_entry(order):
    import block_sparse_video_cube_amd as vsa
    from block_sparse_video_cube_amd import _lib

    lib = _lib.load()
    cases = [((1, 4, 128), (8, 8, 12), True, 11.0), ((2, 1, 64), (5, 6, 7), False, 0.25)]
    for (B, H, D), grid, means, amp in cases:
        wl = workloads.workload("tiny").with_(grid=grid, batch=B, heads=H, head_dim=D)
        inp = workloads.make_inputs(wl)
        # A larger amplitude first, so stale maxima from call 1 would be too
        # large for call 2 if the scratch were not cleared.
        q, k, v = (to_dev(inp[n]) * amp for n in ("q", "k", "v"))
        g = vsa.make_geom(B, H, D, grid)
        d = vsa.geom_dims(g)
        got = outputs(B, H, D, d.n_cubes, d.rows, means)
        st = lib.vsa_quant_fp8_noalloc(g, q.data_ptr(), k.data_ptr(), v.data_ptr(), *[ptr(t) for t in got],
                                       ctypes.c_void_p(vsa._stream()))
        assert st == 0, lib.vsa_status_string(st)
        ref = vsa.quant_fp8(q, k, v, grid, want_means=means)
        torch.cuda.synchronize()
        for a, b in zip(got, ref):
            assert (a is None) == (b is None)
            if a is not None:
                assert torch.equal(a, b)
        print(f"B={B} H={H} D={D} grid={grid}: all outputs identical")


def test_noalloc_rejects_problems_beyond_the_scratch():
    import block_sparse_video_cube_amd as vsa
    from block_sparse_video_cube_amd import _lib

    lib = _lib.load()
    P = 0x10000  # never dereferenced: the size check fails before any launch
    g = vsa.make_geom(4, 129, 128, (4, 4, 4))  # 4 * 129 * 128 > 65536 words
    args = [P] * 9 + [None, None, None]
    assert lib.vsa_quant_fp8_noalloc(g, *args) == _lib.VSA_ERR_SCRATCH
    g_ok = vsa.make_geom(4, 128, 128, (4, 4, 4))
    assert lib.vsa_quant_fp8_noalloc(g_ok, *([None] + [P] * 8 + [None, None, None])) == _lib.VSA_ERR_NULL
