"""GPU parity of the low-precision fine stage (fp8 E4M3 codes, fp8 matrix
products) against the fp64 oracle.

The packed stage (vsa_quant_fp8_packed, vsa_sparse_attn_fwd_fp8_packed) is
held to the same checks: its layouts bit-exact (K codes in compact rows, V
codes in 16-key slots), and its outputs within the bounds of items 2 and 3.

1. The quantizers are bit-exact against the oracle's (O10): codes and scales
   of Q and K per (b, h, cube), of V per (b, h, channel); V's codes in the
   documented tile order (each cube transposed, key k = 32 t + 16 g + 8 h + e
   at position 32 h + 16 t + 8 g + e).  The cube means the same pass writes
   are bit-identical to the pooling kernel's.
2. With Q = 0 every weight is exactly 1, so the fp8 stage must give the mean
   of the dequantized V over the selected valid keys, up to fp32 sums and the
   bf16 output rounding.
3. Against the oracle on the dequantized inputs (the same codes times the same
   scales, in fp64), the only approximation left is the rounding of the
   softmax weights to E4M3.  The stage rounds weights scaled so that a row's
   largest lies in [2^4, 2^8]; a weight p (relative to the row's largest, so
   p <= 1) then rounds with error at most e = max(2^-4 p, 2^-14) (half a step:
   3 mantissa bits; subnormal step 2^-9 before the scaling of at least 2^4),
   and fp32 logits, exp2 and sums add at most 2^-12 p.  As the normaliser sums
   the same rounded weights, O~ - O = sum_k (p~_k - p_k)(v_k - O) / sum p~, so
   every output element obeys |O~ - O| <= sum_k e_k |v_k - O| / (sum p - sum e)
   + 2^-11 sum_k p_k |v_k| / sum p, plus the bf16 rounding 2^-8 |O|, and the
   log-sum-exp |dlse| <= -log(1 - sum e / sum p).  In the mean the weight
   errors do not add up coherently: mean|d| <= 2^-4 mean|ref|.
4. Against the oracle on the original bf16 inputs (looser: the E4M3 rounding
   of Q, K and V adds to P's): mean|d| <= 2^-3 mean|ref|, max|d| <= 2^-2 max|ref|.
"""

import numpy as np
import pytest
import torch

import oracle
import workloads
from tests.gpu_util import assert_close_rel, to_bits, to_dev

pytestmark = pytest.mark.gpu

# Position of key k inside a row of an fp8 V^T tile (the header's layout).
VKEY_POS = np.array([32 * ((k >> 3) & 1) + 16 * (k >> 5) + 8 * ((k >> 4) & 1) + (k & 7) for k in range(64)])

MEAN_REL_DEQ = 2.0 ** -4
MEAN_REL_EXACT = 2.0 ** -3
MAX_REL_EXACT = 2.0 ** -2

CASES = [
    # (B, H, D, grid, k)
    (1, 2, 64, (8, 8, 8), 2),
    (2, 3, 128, (8, 12, 16), 5),
    (1, 2, 128, (9, 14, 13), 4),   # partial cubes on every axis
    (1, 1, 64, (5, 6, 7), 3),
    (1, 1, 128, (8, 8, 12), 12),   # every cube selected
    (1, 2, 128, (8, 8, 8), 1),
]


def oracle_codes(inp, grid):
    valid = oracle.valid_rows(grid)
    qc, kc, vc = (oracle.cube_permute(inp[n], grid) for n in ("q", "k", "v"))
    q8, qs = oracle.quant_cubes(qc, valid)
    k8, ks = oracle.quant_cubes(kc, valid)
    v8, vs = oracle.quant_channels(vc, valid)
    return (q8, qs), (k8, ks), (v8, vs)


def v_tiles(v8: np.ndarray) -> np.ndarray:
    """[B, H, Np, D] codes -> [B, H, Nc, D, 64] tiles in the documented key order."""
    B, Hh, Np, D = v8.shape
    cv = v8.reshape(B, Hh, Np // 64, 64, D).transpose(0, 1, 2, 4, 3)
    out = np.empty_like(cv)
    out[..., VKEY_POS] = cv
    return out


def dequant(codes, scale, per_cube: bool):
    x = oracle.e4m3_decode(codes)
    if per_cube:
        return x * np.repeat(scale.astype(np.float64), 64, axis=2)[..., None]
    return x * scale.astype(np.float64)[:, :, None, :]


def gpu_fp8(inp, grid, idx_np, scale, q_zero=False, packed=False):
    import block_sparse_video_cube_amd as vsa

    q, k, v = (to_dev(inp[n]) for n in ("q", "k", "v"))
    if q_zero:
        q = torch.zeros_like(q)
    q8, qs, k8, ks, v8t, vs, qm, km = vsa.quant_fp8(q, k, v, grid, want_means=True, packed=packed)
    idx = torch.from_numpy(np.ascontiguousarray(idx_np, dtype=np.int32)).to("cuda:0")
    stage = vsa.sparse_attn_fwd_fp8_packed if packed else vsa.sparse_attn_fwd_fp8
    oc, lse = stage(q8, qs, k8, ks, v8t, vs, idx, grid, scale, want_lse=True)
    # The raster-order output is the same values at raster positions.
    o_r, lse_r = stage(q8, qs, k8, ks, v8t, vs, idx, grid, scale, want_lse=True, raster=True)
    assert torch.equal(o_r, vsa.cube_unpermute(oc, grid)) and torch.equal(lse_r, lse)
    # The means for the coarse stage come out of the same pass, bit-identical to the pooling kernel's.
    assert torch.equal(qm, vsa.cube_pool(q, grid)) and torch.equal(km, vsa.cube_pool(k, grid))
    torch.cuda.synchronize()
    codes = tuple(t.cpu().numpy() for t in (q8, qs, k8, ks, v8t, vs))
    return oracle.bf16_to_f64(to_bits(oc)), lse.cpu().numpy().astype(np.float64), codes


def rounding_bound(qd, kd, vd, valid, idx, scale, ref, cubes):
    """Per-element bound of item 3 for the listed (b, h, i) cubes, and the
    per-row log-sum-exp bound."""
    bound = np.full(ref.shape, np.nan)
    lse_bound = np.full(ref.shape[:3], np.nan)
    for b, h, i in cubes:
        keys = np.array([64 * j + l for j in idx[b, h, i] for l in range(64)], dtype=np.int64)
        lg = scale * (qd[b, h, 64 * i:64 * i + 64] @ kd[b, h, keys].T)
        lg[:, ~valid[keys]] = -np.inf
        p = np.exp(lg - lg.max(axis=1, keepdims=True))
        e = np.maximum(2.0 ** -4 * p, np.where(valid[keys], 2.0 ** -14, 0.0)) + 2.0 ** -12 * p
        vv = vd[b, h, keys]
        den = p.sum(axis=1) - e.sum(axis=1)
        lse_bound[b, h, 64 * i:64 * i + 64] = -np.log1p(-e.sum(axis=1) / p.sum(axis=1)) + 2.0 ** -12
        acc = (p @ np.abs(vv)) / p.sum(axis=1, keepdims=True)
        for r in range(64):
            o = ref[b, h, 64 * i + r]
            bound[b, h, 64 * i + r] = (e[r] @ np.abs(vv - o)) / den[r] + 2.0 ** -11 * acc[r] + 2.0 ** -8 * np.abs(o)
    return bound + 1e-7, lse_bound


def select(inp, grid, k):
    valid = oracle.valid_rows(grid)
    return oracle.select_topk(oracle.cube_permute(inp["q"], grid), oracle.cube_permute(inp["k"], grid), valid, k)


def make_case(B, H, D, grid, k, seed):
    wl = workloads.workload("tiny").with_(batch=B, heads=H, head_dim=D, grid=grid, topk=k, seed=seed)
    return wl, workloads.make_inputs(wl)


@pytest.mark.parametrize("B,H,D,grid,k", CASES[:4])
def test_quantizers_bit_exact(B, H, D, grid, k):
    wl, inp = make_case(B, H, D, grid, k, 4000 + D + k)
    idx = select(inp, grid, k)
    _, _, got = gpu_fp8(inp, grid, idx, wl.softmax_scale)
    (q8, qs), (k8, ks), (v8, vs) = oracle_codes(inp, grid)
    valid = oracle.valid_rows(grid)
    assert np.array_equal(got[0][:, :, valid], q8[:, :, valid]) and np.array_equal(got[1], qs)
    assert np.array_equal(got[0][:, :, ~valid], q8[:, :, ~valid])  # padded rows are zero codes
    assert np.array_equal(got[2], k8) and np.array_equal(got[3], ks)
    assert np.array_equal(got[4], v_tiles(v8)) and np.array_equal(got[5], vs)


def test_quantizer_zero_head_and_extremes():
    grid = (8, 8, 8)
    wl, inp = make_case(1, 2, 128, grid, 2, 4100)
    inp["k"][:, :, 1, :] = 0                                   # head 1 all zero: scale 0, codes 0
    inp["v"][:, 5, 0, :] = workloads.round_to_bf16_bits(np.full(128, 3.0e4, np.float32))  # one huge token
    inp["q"][:, 7, 0, :3] = workloads.round_to_bf16_bits(np.array([-1e-30, 1e-38, -0.0], np.float32))
    _, _, got = gpu_fp8(inp, grid, select(inp, grid, 2), wl.softmax_scale)
    (q8, qs), (k8, ks), (v8, vs) = oracle_codes(inp, grid)
    assert np.array_equal(got[0], q8) and np.array_equal(got[1], qs)
    assert np.array_equal(got[2], k8) and np.array_equal(got[3], ks)
    assert np.all(got[3][:, 1] == 0) and np.all(got[2][:, 1] == 0)
    assert np.array_equal(got[4], v_tiles(v8)) and np.array_equal(got[5], vs)


@pytest.mark.parametrize("B,H,D,grid,k", CASES)
def test_uniform_weights_give_mean_of_selected_values(B, H, D, grid, k):
    wl, inp = make_case(B, H, D, grid, k, 4200 + k)
    idx = select(inp, grid, k)
    got, lse, _ = gpu_fp8(inp, grid, idx, wl.softmax_scale, q_zero=True)
    valid = oracle.valid_rows(grid)
    _, _, (v8, vs) = oracle_codes(inp, grid)
    vd = dequant(v8, vs, per_cube=False)
    kd = np.zeros_like(vd)
    ref, ref_lse = oracle.sparse_attention(np.zeros_like(vd), kd, vd, valid, idx, wl.softmax_scale)
    err = np.abs(got - ref)[:, :, valid]
    tol = 2.0 ** -8 * np.abs(ref[:, :, valid]) + 2.0 ** -16 * np.abs(vd).max()
    print(f"uniform weights: max|d| {err.max():.3e}, worst d/tol {np.max(err / tol):.3f}")
    assert np.all(err <= tol)
    assert np.allclose(lse[:, :, valid], ref_lse[:, :, valid], rtol=0, atol=1e-5)


def check_vs_dequantized(inp, grid, idx, scale, cubes=None, what="", packed=False):
    valid = oracle.valid_rows(grid)
    got, lse, _ = gpu_fp8(inp, grid, idx, scale, packed=packed)
    (q8, qs), (k8, ks), (v8, vs) = oracle_codes(inp, grid)
    qd, kd, vd = dequant(q8, qs, True), dequant(k8, ks, True), dequant(v8, vs, False)
    ref, ref_lse = oracle.sparse_attention(qd, kd, vd, valid, idx, scale, cubes)
    B, Hh, Np, _ = ref.shape
    if cubes is None:
        cubes = [(b, h, i) for b in range(B) for h in range(Hh) for i in range(Np // 64)]
    rows = np.zeros((B, Hh, Np), dtype=bool)
    for b, h, i in cubes:
        rows[b, h, 64 * i:64 * i + 64] = valid[64 * i:64 * i + 64]
    bound, lse_bound = rounding_bound(qd, kd, vd, valid, idx, scale, ref, cubes)
    err = np.abs(got - ref)[rows]
    ratio = float(np.max(err / bound[rows]))
    mean_rel = float(err.mean() / np.abs(ref[rows]).mean())
    dl = np.abs(lse[rows] - ref_lse[rows])
    lratio = float(np.max(dl / lse_bound[rows]))
    print(f"{what} vs dequantized: max|d| {err.max():.3e}, worst d/bound {ratio:.3f}, "
          f"mean|d|/mean|ref| {mean_rel:.3e}, max|dlse| {dl.max():.3e}, worst dlse/bound {lratio:.3f}")
    assert np.all(np.isfinite(got[rows]))
    assert ratio <= 1.0
    assert mean_rel <= MEAN_REL_DEQ
    assert lratio <= 1.0
    return got, rows


@pytest.mark.parametrize("B,H,D,grid,k", CASES)
def test_fp8_matches_oracle_on_dequantized_inputs(B, H, D, grid, k):
    wl, inp = make_case(B, H, D, grid, k, 4300 + 7 * k + D)
    check_vs_dequantized(inp, grid, select(inp, grid, k), wl.softmax_scale, what=f"{B}x{H}x{D} {grid} k={k}")


@pytest.mark.parametrize("B,H,D,grid,k", CASES[1:3])
def test_fp8_matches_exact_oracle_loosely(B, H, D, grid, k):
    wl, inp = make_case(B, H, D, grid, k, 4400 + k)
    idx = select(inp, grid, k)
    got, _, _ = gpu_fp8(inp, grid, idx, wl.softmax_scale)
    valid = oracle.valid_rows(grid)
    qc, kc, vc = (oracle.cube_permute(inp[n], grid) for n in ("q", "k", "v"))
    ref, _ = oracle.sparse_attention(qc, kc, vc, valid, idx, wl.softmax_scale)
    assert_close_rel(got[:, :, valid], ref[:, :, valid], "fp8 vs exact", MAX_REL_EXACT, MEAN_REL_EXACT)


@pytest.mark.parametrize("name,head,packed", [("wan1.3b", 0, False), ("720p", 5, False), ("wan14b", 3, False),
                                              ("720p", 9, True), ("wan1.3b", 2, True)])
def test_fp8_full_size_sampled(name, head, packed):
    """One head at the full token grid and top-k; sampled query cubes (packed: the packed stage)."""
    wl = workloads.workload(name)
    full = workloads.make_inputs(wl, heads=[head])
    inp = {n: np.ascontiguousarray(full[n][:, :, [head], :]) for n in ("q", "k", "v")}
    del full
    idx = select(inp, wl.grid, wl.topk)
    nc = oracle.n_cubes(wl.grid)
    cubes = [(0, 0, i) for i in np.linspace(0, nc - 1, 12).astype(int)]
    print(f"[{name}] head {head}: GPU fp8 stage and oracle on {len(cubes)} cubes", flush=True)
    got, rows = check_vs_dequantized(inp, wl.grid, idx, wl.softmax_scale, cubes, what=name, packed=packed)
    valid = oracle.valid_rows(wl.grid)
    qc, kc, vc = (oracle.cube_permute(inp[n], wl.grid) for n in ("q", "k", "v"))
    ref, _ = oracle.sparse_attention(qc, kc, vc, valid, idx, wl.softmax_scale, cubes)
    assert_close_rel(got[rows], ref[rows], f"{name} fp8 vs exact", MAX_REL_EXACT, MEAN_REL_EXACT)


# ------------------------------------------------------------------ packed --
# The packed stage's layouts (vsa_quant_fp8_packed) and the stage on them
# (vsa_sparse_attn_fwd_fp8_packed): tiles of 16-key slots, edge cubes sharing
# tiles (grids with partial cubes) or one cube per tile (full grids).

def compact_rows(x: np.ndarray, grid) -> np.ndarray:
    """[B, H, Np, D] cube-major rows -> the same rows in compact order per cube."""
    order = oracle.compact_order(grid)
    rows = (64 * np.arange(order.shape[0])[:, None] + order).reshape(-1)
    return x[:, :, rows, :]


@pytest.mark.parametrize("B,H,D,grid,k", CASES[:4])
def test_packed_quantizers_bit_exact(B, H, D, grid, k):
    wl, inp = make_case(B, H, D, grid, k, 4500 + D + k)
    idx = select(inp, grid, k)
    _, _, got = gpu_fp8(inp, grid, idx, wl.softmax_scale, packed=True)
    (q8, qs), (k8, ks), (v8, vs) = oracle_codes(inp, grid)
    valid = oracle.valid_rows(grid)
    assert np.array_equal(got[0][:, :, valid], q8[:, :, valid]) and np.array_equal(got[1], qs)
    assert np.array_equal(got[2], compact_rows(k8, grid)) and np.array_equal(got[3], ks)
    assert np.array_equal(got[4], oracle.cube_slots(compact_rows(v8, grid))) and np.array_equal(got[5], vs)


@pytest.mark.parametrize("B,H,D,grid,k", CASES + [(1, 2, 128, (21, 45, 20), 30), (2, 1, 64, (6, 9, 13), 20)])
def test_packed_fp8_matches_oracle_on_dequantized_inputs(B, H, D, grid, k):
    wl, inp = make_case(B, H, D, grid, k, 4600 + 7 * k + D)
    check_vs_dequantized(inp, grid, select(inp, grid, k), wl.softmax_scale, packed=True,
                         what=f"packed {B}x{H}x{D} {grid} k={k}")


@pytest.mark.parametrize("B,H,D,grid,k", CASES[1:4])
def test_packed_uniform_weights_give_mean_of_selected_values(B, H, D, grid, k):
    wl, inp = make_case(B, H, D, grid, k, 4700 + k)
    idx = select(inp, grid, k)
    got, lse, _ = gpu_fp8(inp, grid, idx, wl.softmax_scale, q_zero=True, packed=True)
    valid = oracle.valid_rows(grid)
    _, _, (v8, vs) = oracle_codes(inp, grid)
    vd = dequant(v8, vs, per_cube=False)
    ref, ref_lse = oracle.sparse_attention(np.zeros_like(vd), np.zeros_like(vd), vd, valid, idx, wl.softmax_scale)
    err = np.abs(got - ref)[:, :, valid]
    tol = 2.0 ** -8 * np.abs(ref[:, :, valid]) + 2.0 ** -16 * np.abs(vd).max()
    assert np.all(err <= tol)
    assert np.allclose(lse[:, :, valid], ref_lse[:, :, valid], rtol=0, atol=1e-5)
