"""Pins of the oracle's 8-bit quantization (O10), independent of its code.

- E4M3 values fixed by the OCP 8-bit floating point definition (E4M3FN):
  landmarks (1.0, 448, 2^-6, 2^-9, NaN codes) and the full value table's
  structure;
- round to nearest even against torch's own float8_e4m3fn conversion on a
  large sample, and on hand-picked ties;
- the quantizers: block maxima hit +-448 exactly, dequantized values are
  within half an E4M3 step of the input, zero blocks stay zero.
"""

import numpy as np
import pytest
import torch

import oracle
import workloads


def test_e4m3_landmarks():
    dec = oracle.e4m3_decode
    assert dec(0x38) == 1.0 and dec(0xB8) == -1.0
    assert dec(0x7E) == 448.0 and dec(0xFE) == -448.0
    assert dec(0x08) == 2.0 ** -6          # smallest normal
    assert dec(0x01) == 2.0 ** -9          # smallest subnormal
    assert dec(0x07) == 7 * 2.0 ** -9      # largest subnormal
    assert np.isnan(dec(0x7F)) and np.isnan(dec(0xFF))
    assert dec(0x00) == 0.0 and dec(0x80) == 0.0
    table = dec(np.arange(0x7F))
    assert np.all(np.diff(table) > 0)      # codes 0..126 are strictly increasing
    assert len(table) == 127


def test_e4m3_round_trip_every_code():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    vals = oracle.e4m3_decode(codes).astype(np.float32)
    vals[codes == 0x80] = -0.0
    assert np.array_equal(oracle.e4m3_encode(vals), codes)


def test_e4m3_round_to_nearest_even_ties():
    # midpoints between neighbours: the code with even mantissa wins
    assert oracle.e4m3_encode(np.float32([1.0625]))[0] == 0x38   # 1.0 | 1.125 -> 1.0
    assert oracle.e4m3_encode(np.float32([1.1875]))[0] == 0x3A   # 1.125 | 1.25 -> 1.25
    assert oracle.e4m3_encode(np.float32([432.0]))[0] == 0x7E    # 416 | 448 -> 448 (m = 6)
    assert oracle.e4m3_encode(np.float32([2.0 ** -10]))[0] == 0x00  # 0 | 2^-9 -> 0
    assert oracle.e4m3_encode(np.float32([3 * 2.0 ** -10]))[0] == 0x02  # 2^-9 | 2^-8 -> 2^-8


def test_e4m3_matches_torch_conversion():
    rng = np.random.default_rng(1)
    x = np.concatenate([rng.uniform(-448, 448, 200000), rng.normal(0, 1, 200000),
                        rng.normal(0, 0.01, 200000), [0.0, -0.0, 448.0, -448.0]]).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(oracle.e4m3_encode(x), ref)


@pytest.mark.parametrize("grid", [(8, 8, 8), (5, 6, 7)])
def test_quantizers(grid):
    wl = workloads.workload("tiny").with_(heads=2, head_dim=64, grid=grid)
    inp = workloads.make_inputs(wl)
    valid = oracle.valid_rows(grid)
    xc = oracle.cube_permute(inp["q"], grid)
    x = oracle.bf16_to_f64(xc)
    for codes, scale, per_cube in (oracle.quant_cubes(xc, valid) + (True,),
                                   oracle.quant_channels(xc, valid) + (False,)):
        deq = oracle.e4m3_decode(codes)
        deq = deq * (np.repeat(scale, 64, axis=2)[..., None] if per_cube else scale[:, :, None, :])
        # every block's largest |x| is coded as 448 exactly
        if per_cube:
            blocks = np.abs(oracle.e4m3_decode(codes)).reshape(codes.shape[0], codes.shape[1], -1, 64 * codes.shape[3])
            assert np.all(blocks.max(axis=-1) == 448.0)
        else:
            assert np.all(np.abs(oracle.e4m3_decode(codes)).max(axis=2) == 448.0)
        # within half a step: relative 2^-4 for normals, 2^-10 * scale for subnormals
        err = np.abs(deq - x)[:, :, valid]
        s_b = (np.repeat(scale, 64, axis=2)[..., None] if per_cube else scale[:, :, None, :])
        s_b = np.broadcast_to(s_b, x.shape)[:, :, valid]
        assert np.all(err <= np.maximum(np.abs(x[:, :, valid]) * 2.0 ** -4, s_b * 2.0 ** -10) * (1 + 1e-6))
        assert np.all(codes[:, :, ~valid] == 0)


def test_zero_block_stays_zero():
    grid = (4, 4, 4)
    xc = np.zeros((1, 1, 64, 8), dtype=np.uint16)
    codes, scale = oracle.quant_cubes(xc, oracle.valid_rows(grid))
    assert np.all(codes == 0) and np.all(scale == 0)
