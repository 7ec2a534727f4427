"""Helpers shared by the GPU parity tests (tensor transfer and comparisons)."""

import numpy as np
import torch

import oracle

# Output tolerance of bf16 results against the fp64 oracle, over valid elements.
MAX_ABS = 2e-2
MEAN_ABS = 2e-3


def to_dev(bits: np.ndarray) -> torch.Tensor:
    """uint16 bf16 bit patterns -> torch.bfloat16 on cuda:0."""
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to("cuda:0")


def to_bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu").contiguous().view(torch.int16).numpy().view(np.uint16)


def bf16_f64(t: torch.Tensor) -> np.ndarray:
    return oracle.bf16_to_f64(to_bits(t))


def assert_close(got: np.ndarray, ref: np.ndarray, what: str, max_abs=MAX_ABS, mean_abs=MEAN_ABS):
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    err = np.abs(got - ref)
    mx, mn = float(err.max()), float(err.mean())
    print(f"{what}: max|d|={mx:.3e} mean|d|={mn:.3e} n={err.size}")
    assert mx <= max_abs and mn <= mean_abs, f"{what}: max {mx:.3e} mean {mn:.3e}"


def topk_valid_under(scores: np.ndarray, chosen: np.ndarray, k: int, rel: float = 1e-5) -> bool:
    """Is `chosen` (k distinct indices) a valid top-k of `scores` up to rel * max|s|?"""
    chosen = np.asarray(chosen)
    if len(set(chosen.tolist())) != k or np.any(np.diff(chosen) <= 0):
        return False
    kth = np.sort(scores)[::-1][k - 1]
    tol = rel * max(1.0, float(np.abs(scores).max()))
    mask = np.zeros(scores.size, dtype=bool)
    mask[chosen] = True
    return bool(np.all(scores[mask] >= kth - tol) and np.all(scores[~mask] <= kth + tol))


def assert_close_rel(got: np.ndarray, ref: np.ndarray, what: str, max_rel: float, mean_rel: float):
    """Errors measured against the scale of the reference tensor itself:
    max|d| <= max_rel * max|ref| and mean|d| <= mean_rel * mean|ref|."""
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    err = np.abs(got - ref)
    mx, mn = float(err.max()), float(err.mean())
    rmx, rmn = float(np.abs(ref).max()), float(np.abs(ref).mean())
    print(f"{what}: max|d|={mx:.3e} ({mx / max(rmx, 1e-30):.2e} of max|ref| {rmx:.3e}), "
          f"mean|d|={mn:.3e} ({mn / max(rmn, 1e-30):.2e} of mean|ref| {rmn:.3e})")
    assert mx <= max_rel * rmx and mn <= mean_rel * rmn, f"{what}: max {mx:.3e} mean {mn:.3e}"
