"""Seeded synthetic inputs for cube block-sparse video attention.

This module is shared by the fp64 oracle tests, the GPU parity tests and the
benchmark.  It holds no arithmetic of the attention method itself: it only
draws random numbers, shapes them like the attention inputs of the video
transformers the pages discuss, and rounds them once to bf16 (round to nearest
even).  Both sides receive the same uint16 bit patterns.

Shapes.  The latent grids follow the Wan2.1 / Wan2.2 video sizes named on the
pages (FastVideo docs "Distillation", section "Model Overview": 61x448x832
training shape; the dataset "Wan-Syn_77x448x832_600k"; the SparkDiffusion
article's 720p runs), mapped to a latent token grid by
t' = (frames - 1) / 4 + 1, h' = height / 16, w' = width / 16.
Sparsities 0.8 / 0.9 / 0.97 are those the pages give for VSA and RoLA
(FastVideo sparse-distillation article, section "2. 视频稀疏注意力VSA";
SparkDiffusion article, paragraphs 2-3).

Layout of every tensor handed to the library: [batch, tokens, heads, head_dim]
with tokens in raster order (t slowest, x fastest), bf16 bit patterns as
numpy uint16.

Every tensor of one head is drawn from its own counter-keyed stream,
SeedSequence([seed, tensor_id, b, h]), so that a sampled check can regenerate
a single head without drawing the whole tensor.
"""

from __future__ import annotations

import concurrent.futures
import dataclasses
import os
from fractions import Fraction
from typing import Dict, Optional, Tuple

import numpy as np

__all__ = [
    "Workload",
    "WORKLOADS",
    "workload",
    "topk_for_sparsity",
    "round_to_bf16_bits",
    "bf16_bits_to_f32",
    "make_inputs",
    "make_head",
    "make_integer_inputs",
    "make_tie_inputs",
]

# Tensor ids used as stream keys.
_TID = {"q": 1, "k": 2, "v": 3}


@dataclasses.dataclass(frozen=True)
class Workload:
    """One attention-layer workload: sizes, k and the input recipe."""

    name: str
    batch: int
    heads: int
    head_dim: int
    grid: Tuple[int, int, int]  # valid latent grid (T, H, W)
    topk: int
    sparsity: Optional[float]
    seed: int
    recipe: str  # "normal", "head_scale", "sinusoid"
    linear: bool = False
    # Block pattern: "topk" (coarse-stage selection) or "sta" (static sliding
    # tile window of `window` cubes, see oracle O8).
    pattern: str = "topk"
    window: Optional[Tuple[int, int, int]] = None

    @property
    def tokens(self) -> int:
        t, h, w = self.grid
        return t * h * w

    @property
    def padded_grid(self) -> Tuple[int, int, int]:
        return tuple(((d + 3) // 4) * 4 for d in self.grid)

    @property
    def n_cubes(self) -> int:
        tp, hp, wp = self.padded_grid
        return (tp // 4) * (hp // 4) * (wp // 4)

    @property
    def rows(self) -> int:
        return self.n_cubes * 64

    @property
    def softmax_scale(self) -> float:
        return 1.0 / float(np.sqrt(self.head_dim))

    @property
    def blocks(self) -> int:
        """Number of 64x64 blocks the fine stage computes."""
        return self.batch * self.heads * self.n_cubes * self.topk

    @property
    def fine_flops(self) -> int:
        """QK^T and PV flops over the computed blocks: 4 * 64 * 64 * D each."""
        return self.blocks * 4 * 64 * 64 * self.head_dim

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


def topk_for_sparsity(sparsity, n_cubes: int) -> int:
    """k = ceil((1 - s) * Nc) in exact rational arithmetic.

    The pages state the kept fraction as one minus the sparsity (FastVideo
    sparse-distillation article, section "2. 视频稀疏注意力VSA": sparsity
    0.8-0.9 keeps 10-20 % of the weights; SparkDiffusion article paragraph 2:
    97 % sparsity keeps 3 % of the blocks).  Rounding up keeps at least that
    fraction.  The sparsity is read as a decimal string so that 0.9 means
    9/10 exactly.
    """
    s = Fraction(str(sparsity))
    keep = (1 - s) * n_cubes
    k = -((-keep.numerator) // keep.denominator)
    return int(max(1, min(n_cubes, k)))


WORKLOADS: Dict[str, Workload] = {
    # Tiny sanity case: 8 full cubes, k = 2.
    "tiny": Workload("tiny", 1, 2, 64, (8, 8, 8), 2, 0.75, 1000, "normal"),
    # Wan2.1-1.3B layer at 61x448x832 (latent 16x28x52), sparsity 0.8.
    "wan1.3b": Workload("wan1.3b", 1, 12, 128, (16, 28, 52), 73, 0.8, 1001, "head_scale"),
    # Wan2.1-14B layer at 77x448x832 (latent 20x28x52), sparsity 0.9.
    "wan14b": Workload("wan14b", 1, 40, 128, (20, 28, 52), 46, 0.9, 1002, "sinusoid"),
    # 720P layer: latent 21x45x80, zero padded to 24x48x80, sparsity 0.9.
    "720p": Workload("720p", 1, 40, 128, (21, 45, 80), 144, 0.9, 1003, "normal"),
    # High-sparsity hybrid with the linear branch, sparsity 0.97.
    "hybrid": Workload("hybrid", 2, 12, 128, (16, 28, 52), 11, 0.97, 1004, "normal", linear=True),
    # Sliding-tile pattern on the Wan2.1-1.3B layer: a 3x3x3-cube window
    # (k = 27 of 364 cubes).  The pages name STA but give no window size.
    "sta": Workload("sta", 1, 12, 128, (16, 28, 52), 27, None, 1005, "head_scale", pattern="sta",
                    window=(3, 3, 3)),
}


def workload(name: str) -> Workload:
    return WORKLOADS[name]


# --------------------------------------------------------------------------
# bf16 bit patterns (input preparation only)
# --------------------------------------------------------------------------

def round_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit pattern, round to nearest, ties to even."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


# --------------------------------------------------------------------------
# Generators
# --------------------------------------------------------------------------

def _stream(seed: int, tid: int, b: int, h: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, tid, b, h])))


def _head_scales(wl: Workload) -> np.ndarray:
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([wl.seed, 99])))
    return rng.uniform(0.5, 2.0, size=wl.heads).astype(np.float32)


def _sinusoid_field(wl: Workload, h: int) -> np.ndarray:
    """[S, D] fp32 smooth low-frequency 3D sinusoid for head h (amplitude 1).

    For each (head, d): sin(2 pi (a t/T + b y/H + c x/W) + phase), with
    integer frequencies a, b, c in {0, 1, 2} (not all zero) and a uniform
    phase, all drawn from the workload seed.
    """
    T, H, W = wl.grid
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([wl.seed, 98, h])))
    D = wl.head_dim
    freqs = rng.integers(0, 3, size=(D, 3))
    zero = np.all(freqs == 0, axis=1)
    freqs[zero, 0] = 1
    phase = rng.uniform(0.0, 2.0 * np.pi, size=D)
    t = np.arange(T, dtype=np.float64)[:, None, None] / T
    y = np.arange(H, dtype=np.float64)[None, :, None] / H
    x = np.arange(W, dtype=np.float64)[None, None, :] / W
    out = np.empty((T * H * W, D), dtype=np.float32)
    for d in range(D):
        a, b, c = freqs[d]
        arg = 2.0 * np.pi * (a * t + b * y + c * x) + phase[d]
        out[:, d] = np.sin(arg).reshape(-1)
    return out


def make_head(wl: Workload, name: str, b: int, h: int) -> np.ndarray:
    """One head of one input tensor: [S, D] bf16 bits."""
    S, D = wl.tokens, wl.head_dim
    x = _stream(wl.seed, _TID[name], b, h).standard_normal((S, D), dtype=np.float32)
    if wl.recipe == "head_scale":
        x *= _head_scales(wl)[h]
    elif wl.recipe == "sinusoid" and name in ("q", "k"):
        x += _sinusoid_field(wl, h)
    elif wl.recipe != "normal" and wl.recipe not in ("head_scale", "sinusoid"):
        raise ValueError(f"unknown recipe {wl.recipe!r}")
    return round_to_bf16_bits(x)


def make_inputs(wl: Workload, heads=None) -> Dict[str, np.ndarray]:
    """q, k, v as [B, S, heads, D] uint16 (bf16 bits).

    heads: optional list of head indices to draw (the others stay zero); used
    for sampled checks at full size.
    """
    B, S, Hh, D = wl.batch, wl.tokens, wl.heads, wl.head_dim
    hs = range(Hh) if heads is None else heads
    out = {name: np.zeros((B, S, Hh, D), dtype=np.uint16) for name in ("q", "k", "v")}

    def fill(job):
        name, b, h = job
        out[name][b, :, h, :] = make_head(wl, name, b, h)

    # Every head comes from its own stream, so the heads can be drawn in any
    # order (and in parallel threads) with the same result.
    jobs = [(name, b, h) for name in ("q", "k", "v") for b in range(B) for h in hs]
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        list(ex.map(fill, jobs))
    return out


def make_integer_inputs(wl: Workload) -> Dict[str, np.ndarray]:
    """Integer-valued variant: q, k i.i.d. uniform over {-2, ..., 2}, v ~ N(0, 1).

    With such inputs every cube sum, every power-of-two mean and every pooled
    dot product is exact in fp32, so block selection can be compared bit for
    bit.
    """
    B, S, Hh, D = wl.batch, wl.tokens, wl.heads, wl.head_dim
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([wl.seed, 7])))
    q = rng.integers(-2, 3, size=(B, S, Hh, D)).astype(np.float32)
    k = rng.integers(-2, 3, size=(B, S, Hh, D)).astype(np.float32)
    v = rng.standard_normal((B, S, Hh, D), dtype=np.float32)
    return {"q": round_to_bf16_bits(q), "k": round_to_bf16_bits(k), "v": round_to_bf16_bits(v)}


def make_tie_inputs(wl: Workload, kind: str) -> Dict[str, np.ndarray]:
    """Adversarial tie cases built on the integer variant.

    kind = "zero_k": K identically zero, so every block score ties.
    kind = "periodic_k": K repeats along x with a period of 8 tokens
    (k[t, y, x] = k[t, y, x mod 8]), so many key regions carry identical
    values and their scores tie exactly.
    """
    inp = make_integer_inputs(wl)
    if kind == "zero_k":
        inp["k"][:] = 0
        return inp
    if kind != "periodic_k":
        raise ValueError(kind)
    T, H, W = wl.grid
    k = inp["k"].reshape(wl.batch, T, H, W, wl.heads, wl.head_dim)
    for x in range(8, W):
        k[:, :, :, x] = k[:, :, :, x % 8]
    inp["k"] = k.reshape(wl.batch, T * H * W, wl.heads, wl.head_dim)
    return inp
