"""GPU parity of the packed fine stage and its layouts.

- Compact and slot permutes (vsa_cube_permute TOKEN_COMPACT / DIM_SLOTS,
  vsa_cube_permute_pool_compact): bit-exact against the oracle's O12 layouts;
  the pooled means bit-identical to vsa_cube_permute_pool's.
- vsa_sparse_attn_fwd_packed against the oracle's fine stage (O5) on grids
  whose edge cubes hold 1..3 valid tokens per axis (so tiles mix one-, two-
  and four-slot cubes), D = 64 and 128, k = 1, k = Nc, raster and cube-major.
- The raster and cube-major forms are bit-identical (output and lse); on a
  grid without padding the packed stage is bit-identical to the unpacked one.
- The packing plan in the workspace holds every selected cube's valid keys
  exactly once, and the launch order of each head sorts its query cubes by
  tile count (most first), then by the mean index of the cubes with a tile of
  their own (ascending and descending in turn over the occupied tile counts),
  then by cube; past 4096 query cubes per head (tile count only) it is a
  permutation with the most tiles first, and the stage still matches the
  oracle.
"""

import numpy as np
import pytest
import torch

import oracle
import workloads
from tests.gpu_util import assert_close, bf16_f64, to_bits, to_dev

pytestmark = pytest.mark.gpu

GRIDS = [(5, 6, 7), (9, 6, 12), (2, 3, 5), (6, 9, 13), (21, 45, 20), (8, 8, 8)]


def inputs(grid, D, heads=2, batch=1, seed=0):
    wl = workloads.workload("tiny").with_(grid=grid, head_dim=D, heads=heads, batch=batch, seed=1000 + seed)
    return wl, workloads.make_inputs(wl)


@pytest.mark.parametrize("grid", GRIDS)
@pytest.mark.parametrize("D", [64, 128])
def test_compact_and_slot_permutes_bit_exact(grid, D):
    import block_sparse_video_cube_amd as vsa

    wl, inp = inputs(grid, D)
    k = to_dev(inp["k"])
    ref = oracle.cube_permute_compact(inp["k"], grid)
    assert np.array_equal(to_bits(vsa.cube_permute(k, grid, layout="compact")), ref)
    assert np.array_equal(to_bits(vsa.cube_permute(k, grid, layout="slots")), oracle.cube_slots(ref))
    kcc, mean_c = vsa.cube_permute_pool(k, grid, compact=True)
    _, mean = vsa.cube_permute_pool(k, grid)
    assert np.array_equal(to_bits(kcc), ref)
    assert torch.equal(mean_c, mean)


def random_lists(wl, topk, rng):
    """Ascending distinct block lists [B, H, Nc, topk]."""
    nc = wl.n_cubes
    idx = np.empty((wl.batch, wl.heads, nc, topk), dtype=np.int32)
    for b in range(wl.batch):
        for h in range(wl.heads):
            for i in range(nc):
                idx[b, h, i] = np.sort(rng.choice(nc, size=topk, replace=False))
    return idx


def run_packed(vsa, inp, wl, idx_d, raster):
    q = to_dev(inp["q"])
    kc = vsa.cube_permute(to_dev(inp["k"]), wl.grid, layout="compact")
    vs = vsa.cube_permute(to_dev(inp["v"]), wl.grid, layout="slots")
    qin = q if raster else vsa.cube_permute(q, wl.grid)
    return vsa.sparse_attn_fwd_packed(qin, kc, vs, idx_d, wl.grid, wl.softmax_scale, want_lse=True, raster=raster)


PACKED_CASES = [
    ((5, 6, 7), 64, 3), ((5, 6, 7), 128, 1), ((9, 6, 12), 128, 7), ((2, 3, 5), 128, 1),
    ((6, 9, 13), 64, 20), ((6, 9, 13), 128, 48), ((21, 45, 20), 128, 36), ((8, 8, 8), 128, 3),
]


@pytest.mark.parametrize("grid,D,topk", PACKED_CASES)
def test_packed_fine_stage_matches_oracle(grid, D, topk):
    import block_sparse_video_cube_amd as vsa

    wl, inp = inputs(grid, D, heads=2, batch=2, seed=topk)
    rng = np.random.default_rng(topk)
    idx = random_lists(wl, min(topk, wl.n_cubes), rng)
    idx_d = torch.from_numpy(idx).to("cuda:0")
    o, lse = run_packed(vsa, inp, wl, idx_d, raster=True)
    oc, lse_c = run_packed(vsa, inp, wl, idx_d, raster=False)
    torch.cuda.synchronize()
    # Raster and cube-major forms: the same tiles in the same order.
    assert torch.equal(vsa.cube_unpermute(oc, wl.grid), o)
    assert torch.equal(lse, lse_c)
    valid = oracle.valid_rows(wl.grid)
    qc, kc, vc = (oracle.cube_permute(inp[n], wl.grid) for n in ("q", "k", "v"))
    ref, ref_lse = oracle.sparse_attention(qc, kc, vc, valid, idx, wl.softmax_scale)
    assert_close(bf16_f64(oc)[:, :, valid], ref[:, :, valid], f"packed {grid} D={D} k={topk}")
    err = np.abs(lse.cpu().numpy()[:, :, valid] - ref_lse[:, :, valid]).max()
    print(f"lse max|d| = {err:.3e}")
    assert err <= 4.5e-3


@pytest.mark.parametrize("grid,D", [((5, 6, 7), 128), ((9, 6, 12), 64), ((2, 3, 5), 128)])
def test_packed_every_cube_selected(grid, D):
    # k = Nc: dense attention over all valid keys; the plan packs every edge cube.
    import block_sparse_video_cube_amd as vsa

    wl, inp = inputs(grid, D)
    nc = wl.n_cubes
    idx = np.broadcast_to(np.arange(nc, dtype=np.int32), (1, wl.heads, nc, nc)).copy()
    o, _ = run_packed(vsa, inp, wl, torch.from_numpy(idx).to("cuda:0"), raster=True)
    valid = oracle.valid_rows(wl.grid)
    qc, kc, vc = (oracle.cube_permute(inp[n], wl.grid) for n in ("q", "k", "v"))
    ref, _ = oracle.sparse_attention(qc, kc, vc, valid, idx, wl.softmax_scale)
    ref_tok = oracle.cube_unpermute(np.nan_to_num(ref), wl.grid)
    assert_close(bf16_f64(o), ref_tok, f"packed dense {grid} D={D}")


@pytest.mark.parametrize("D", [64, 128])
def test_packed_full_grid_bit_identical_to_unpacked(D):
    # Without padded cubes every tile is one whole cube in list order, so the
    # packed stage does exactly the unpacked stage's arithmetic.
    import block_sparse_video_cube_amd as vsa

    wl, inp = inputs((8, 12, 16), D)
    idx = torch.from_numpy(random_lists(wl, 5, np.random.default_rng(1))).to("cuda:0")
    q = to_dev(inp["q"])
    kc = vsa.cube_permute(to_dev(inp["k"]), wl.grid)
    vt = vsa.cube_permute(to_dev(inp["v"]), wl.grid, layout="dim")
    o_ref, lse_ref = vsa.sparse_attn_fwd_raster(q, kc, vt, idx, wl.grid, wl.softmax_scale, want_lse=True)
    o, lse = run_packed(vsa, inp, wl, idx, raster=True)
    assert torch.equal(o, o_ref)
    assert torch.equal(lse, lse_ref)


def test_packing_plan_covers_every_selected_key_once():
    import block_sparse_video_cube_amd as vsa

    grid, D = (9, 6, 12), 128
    wl, inp = inputs(grid, D)
    topk = 11
    idx = random_lists(wl, topk, np.random.default_rng(5))
    idx[0, 1, 3, :4] = idx[0, 1, 3, 4]  # duplicates are computed (and packed) once per entry
    idx_d = torch.from_numpy(idx).to("cuda:0")
    g = vsa.make_geom(1, wl.heads, D, grid)
    ws = torch.zeros(vsa.packed_workspace_bytes(g, topk), dtype=torch.uint8, device="cuda:0")
    run_q = to_dev(inp["q"])
    kc = vsa.cube_permute(to_dev(inp["k"]), grid, layout="compact")
    vs = vsa.cube_permute(to_dev(inp["v"]), grid, layout="slots")
    vsa.sparse_attn_fwd_packed(run_q, kc, vs, idx_d, grid, workspace=ws)
    words = ws.view(torch.int32).cpu().numpy()
    nplan = wl.heads * wl.n_cubes * (topk + 1) * 4
    plan = words[:nplan].reshape(1, wl.heads, wl.n_cubes, topk + 1, 4)
    order = words[nplan:nplan + wl.heads * wl.n_cubes].reshape(wl.heads, wl.n_cubes)
    counts = oracle.valid_rows(grid).reshape(-1, 64).sum(axis=1)
    for h in range(wl.heads):
        for i in range(wl.n_cubes):
            row = plan[0, h, i]
            ntiles = int(row[0, 0])
            # Word 1: the mean index of the list's cubes with three or four slots.
            own = [int(j) for j in idx[0, h, i] if counts[j] > 32]
            assert row[0, 1] == (sum(own) // len(own) if own else 0), (h, i)
            slots = [int(c) for c in row[1:1 + ntiles].reshape(-1) if c != 0]
            got = sorted((c >> 8, (c >> 5) & 3, c & 31) for c in slots)
            want = sorted((int(j), sc, min(16, int(counts[j]) - 16 * sc))
                          for j in idx[0, h, i] for sc in range((int(counts[j]) + 15) // 16))
            assert got == want, (h, i)
            slots_of = [(int(counts[j]) + 15) // 16 for j in idx[0, h, i]]
            nb = sum(s >= 3 for s in slots_of)
            assert ntiles == nb + (sum(s == 2 for s in slots_of) + 1) // 2 + (sum(s == 1 for s in slots_of) + 3) // 4
        # The launch order: tile count (most first), then word 1 ascending on
        # the largest occupied count, descending on the next, and so on, then cube.
        nt = plan[0, h, :, 0, 0].astype(int)
        turn = {t: r % 2 for r, t in enumerate(sorted(set(nt.tolist()), reverse=True))}
        key = [(-nt[i], -plan[0, h, i, 0, 1] if turn[nt[i]] else plan[0, h, i, 0, 1], i) for i in range(wl.n_cubes)]
        assert order[h].tolist() == sorted(range(wl.n_cubes), key=lambda i: key[i]), h


def test_packed_stage_past_the_sorted_order_limit():
    """9537 query cubes per head: the launch order falls back to tile counts only."""
    import block_sparse_video_cube_amd as vsa

    grid, D, topk = (130, 66, 66), 64, 3
    wl, inp = inputs(grid, D, heads=1, seed=7)
    assert wl.n_cubes == 9537
    idx = random_lists(wl, topk, np.random.default_rng(8))
    idx_d = torch.from_numpy(idx).to("cuda:0")
    g = vsa.make_geom(1, 1, D, grid)
    ws = torch.zeros(vsa.packed_workspace_bytes(g, topk), dtype=torch.uint8, device="cuda:0")
    kc = vsa.cube_permute(to_dev(inp["k"]), grid, layout="compact")
    vs = vsa.cube_permute(to_dev(inp["v"]), grid, layout="slots")
    print("[packed, 9537 cubes] fine stage", flush=True)
    qc_d = vsa.cube_permute(to_dev(inp["q"]), grid)
    oc, _ = vsa.sparse_attn_fwd_packed(qc_d, kc, vs, idx_d, grid, wl.softmax_scale, workspace=ws, raster=False)
    words = ws.view(torch.int32).cpu().numpy()
    nplan = wl.n_cubes * (topk + 1) * 4
    plan = words[:nplan].reshape(wl.n_cubes, topk + 1, 4)
    order = words[nplan:nplan + wl.n_cubes]
    assert sorted(order.tolist()) == list(range(wl.n_cubes))
    assert np.all(np.diff(plan[order, 0, 0]) <= 0)
    cubes = [0, 1, 16, 288, 4000, 9520, 9536]
    valid = oracle.valid_rows(grid)
    qc, kc_o, vc = (oracle.cube_permute(inp[n], grid) for n in ("q", "k", "v"))
    ref, _ = oracle.sparse_attention(qc, kc_o, vc, valid, idx, wl.softmax_scale, cubes=[(0, 0, i) for i in cubes])
    rows = np.zeros(wl.rows, dtype=bool)
    for i in cubes:
        rows[64 * i:64 * i + 64] = True
    rows &= valid
    assert_close(bf16_f64(oc)[:, :, rows], ref[:, :, rows], "packed stage, 9537 cubes")
