"""Seeded synthetic inputs for block-sparse video attention.

This module only *draws* inputs.  It holds none of the method's arithmetic
(no pooling, scoring, selection or attention), so that both the HIP path and
the CPU oracle can be fed the very same arrays without sharing any code that
computes a result.

Recipe (one field per batch, head and channel):

* ``z ~ N(0, 1)`` on the latent grid padded by ``r = ceil(4*sigma)`` tokens on
  every side of t, h and w;
* a separable, normalised 1-D Gaussian (taps proportional to
  ``exp(-k^2 / (2 sigma^2))`` for ``|k| <= r``, summing to 1) is applied along
  w, then h, then t, keeping only the "valid" part, so the result has exactly
  the grid's size and no boundary effects;
* ``Q = 4 * smoothed`` (reading A, the literal one) or
  ``Q = 4 * smoothed / std_theory`` (reading B: the field re-standardised to
  unit variance with its exact theoretical standard deviation
  ``sqrt(prod_axes sum_k w_k^2)``);
* ``K = Q + 0.5 * N(0, 1)`` with independent noise, ``V ~ N(0, 1)``;
* tokens are then put in tile-major order: frame-block outermost, then tile
  row, then tile column, then row-major inside the ``tile_t x tile_h x tile_w``
  tile, so that block ``b`` is tokens ``[64 b, 64 b + 64)``; on a grid that is not
  a whole number of tiles the last tiles are partial and their slots beyond the
  grid hold zeros;
* finally the arrays are cast to the workload's dtype (the cast values are
  what every consumer sees).

Random streams: every (tensor, batch, head) draws from its own PCG64 stream
seeded by ``SeedSequence(seed, spawn_key=(tensor, batch, head))`` with tensor
0 = Q noise, 1 = K noise, 2 = V.  Per-head thresholds, when a workload jitters
them, come from the stream ``spawn_key=(3,)`` as ``U(lo, hi)`` in head order.
Independent streams let the draws run on several threads and still be
reproducible bit for bit.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field, replace
from typing import Optional, Tuple

import numpy as np
import torch

__all__ = ["Workload", "WORKLOADS", "make_inputs", "gaussian_taps", "tile_major"]


@dataclass(frozen=True)
class Workload:
    """One synthetic configuration of the attention layer."""

    name: str
    batch: int
    heads: int
    head_dim: int
    grid: Tuple[int, int, int]            # latent grid (T, H, W) in tokens
    dtype: str                            # "f32" | "bf16"
    sigma: float                          # Gaussian smoothing width in tokens
    threshold: float                      # CDF mass kept per query block
    head_threshold_range: Optional[Tuple[float, float]] = None  # per-head U(lo, hi)
    window: Tuple[int, int, int] = (-1, -1, -1)                 # radii in blocks, <0 = off
    tile: Tuple[int, int, int] = (1, 8, 8)
    seed: int = 0
    description: str = field(default="", compare=False)

    @property
    def tokens(self) -> int:
        t, h, w = self.grid
        return t * h * w

    @property
    def block_grid(self) -> Tuple[int, int, int]:
        return tuple(-(-g // s) for g, s in zip(self.grid, self.tile))

    @property
    def partial(self) -> bool:
        return any(g % s for g, s in zip(self.grid, self.tile))

    @property
    def slots(self) -> int:
        """Token slots of a head in tile-major order (nB * 64, padding included)."""
        return self.blocks * 64

    @property
    def blocks(self) -> int:
        a, b, c = self.block_grid
        return a * b * c

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


# The five workloads: a tiny fp32 case and four video-DiT-sized bf16 layers
# (sizes of a Wan2.1-1.3B 480p, a Wan2.1-14B 720p, a HunyuanVideo 720p and a
# long-video layer, grids rounded to whole 8x8 tiles).
WORKLOADS = {
    "tiny_f32": Workload(
        "tiny_f32", 1, 1, 64, (4, 16, 16), "f32", 2.0, 0.9,
        description="1 head, d=64, grid 4x16x16 (1,024 tokens, 16 blocks), fp32, thr 0.9"),
    "wan13b_480p": Workload(
        "wan13b_480p", 1, 12, 128, (20, 32, 48), "bf16", 2.0, 0.9,
        description="12 heads, d=128, grid 20x32x48 (30,720 tokens, 480 blocks), bf16, thr 0.9"),
    "wan14b_720p": Workload(
        "wan14b_720p", 1, 40, 128, (21, 48, 80), "bf16", 3.0, 0.9,
        description="40 heads, d=128, grid 21x48x80 (80,640 tokens, 1,260 blocks), bf16, thr 0.9"),
    "hunyuan_720p": Workload(
        "hunyuan_720p", 1, 24, 128, (32, 48, 80), "bf16", 2.0, 0.8, window=(1, 1, 1),
        description="24 heads, d=128, grid 32x48x80 (122,880 tokens, 1,920 blocks), bf16, "
                    "thr 0.8 united with a +-1 frame / +-1 tile window"),
    "long_video": Workload(
        "long_video", 1, 12, 128, (64, 48, 80), "bf16", 4.0, 0.7, head_threshold_range=(0.6, 0.8),
        description="12 heads, d=128, grid 64x48x80 (245,760 tokens, 3,840 blocks), bf16, "
                    "per-head thr ~ U(0.6, 0.8)"),
}


def gaussian_taps(sigma: float) -> np.ndarray:
    """Normalised 1-D Gaussian taps for |k| <= ceil(4 sigma), in float64."""
    r = int(math.ceil(4.0 * sigma))
    k = np.arange(-r, r + 1, dtype=np.float64)
    w = np.exp(-(k * k) / (2.0 * sigma * sigma))
    return w / w.sum()


def _smooth_valid(x: torch.Tensor, taps: np.ndarray) -> torch.Tensor:
    """Separable 'valid' correlation of x [C, T+2r, H+2r, W+2r] with taps on the last 3 axes."""
    w = torch.tensor(taps, dtype=x.dtype).view(1, 1, -1)
    n = len(taps) - 1
    c, t, h, ww = x.shape
    y = torch.nn.functional.conv1d(x.reshape(-1, 1, ww), w).view(c, t, h, ww - n)
    y = y.permute(0, 1, 3, 2).reshape(-1, 1, h)
    y = torch.nn.functional.conv1d(y, w).view(c, t, ww - n, h - n)
    y = y.permute(0, 2, 3, 1).reshape(-1, 1, t)
    y = torch.nn.functional.conv1d(y, w).view(c, ww - n, h - n, t - n)
    return y.permute(0, 3, 2, 1).contiguous()          # [C, T, H, W]


def tile_major(x: torch.Tensor, grid, tile) -> torch.Tensor:
    """[..., d, T, H, W] field -> [..., nB * V, d] tokens in tile-major order.  When the
    grid is not a whole number of tiles, the last tile along an axis is partial and its
    slots beyond the grid hold zeros (padding)."""
    t, h, w = grid
    tt, th, tw = tile
    pt, ph, pw = (-(-t // tt)) * tt, (-(-h // th)) * th, (-(-w // tw)) * tw
    if (pt, ph, pw) != (t, h, w):
        x = torch.nn.functional.pad(x, (0, pw - w, 0, ph - h, 0, pt - t))
        t, h, w = pt, ph, pw
    lead = x.shape[:-4]
    d = x.shape[-4]
    x = x.reshape(*lead, d, t // tt, tt, h // th, th, w // tw, tw)
    nl = len(lead)
    perm = list(range(nl)) + [nl + i for i in (1, 3, 5, 2, 4, 6, 0)]
    return x.permute(*perm).reshape(*lead, t * h * w, d)


def _stream(seed: int, *key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=key)))


def head_thresholds(wl: Workload) -> np.ndarray:
    """Per-head CDF thresholds (float32) for the workload."""
    if wl.head_threshold_range is None:
        return np.full(wl.heads, wl.threshold, dtype=np.float32)
    lo, hi = wl.head_threshold_range
    return _stream(wl.seed, 3).uniform(lo, hi, size=wl.heads).astype(np.float32)


def make_inputs(wl: Workload, reading: str = "A", threads: Optional[int] = None):
    """Return (q, k, v, thresholds) as CPU torch tensors [B, H, N, d] in the workload dtype.

    ``reading`` selects the Q amplitude: "A" (smoothed field times 4) or "B"
    (smoothed field re-standardised to unit variance, times 4).  ``"page"``
    is the variant with unit-variance field times 1.4.
    """
    if reading not in ("A", "B", "page"):
        raise ValueError(f"unknown reading {reading!r}")
    B, H, d = wl.batch, wl.heads, wl.head_dim
    T, Hh, W = wl.grid
    taps = gaussian_taps(wl.sigma)
    r = (len(taps) - 1) // 2
    amp = 4.0
    if reading in ("B", "page"):
        std = math.sqrt(float(np.sum(taps * taps)) ** 3)
        amp = (4.0 if reading == "B" else 1.4) / std
    tdt = torch.float32 if wl.dtype == "f32" else torch.bfloat16
    N = wl.slots                      # tile-major slots (== tokens for whole tiles)
    q = torch.empty(B, H, N, d, dtype=tdt)
    k = torch.empty(B, H, N, d, dtype=tdt)
    v = torch.empty(B, H, N, d, dtype=tdt)
    threads = threads or min(16, os.cpu_count() or 1)
    pad = (d, T + 2 * r, Hh + 2 * r, W + 2 * r)

    def draw(job):
        tensor, b, h = job
        g = _stream(wl.seed, tensor, b, h)
        if tensor == 0:
            return g.standard_normal(pad, dtype=np.float32)
        return g.standard_normal((d, T, Hh, W), dtype=np.float32)

    heads = [(b, h) for b in range(B) for h in range(H)]
    group = max(1, threads // 3)
    with ThreadPoolExecutor(threads) as ex:
        for i in range(0, len(heads), group):
            chunk = heads[i:i + group]
            jobs = [(t, b, h) for (b, h) in chunk for t in (0, 1, 2)]
            arrays = list(ex.map(draw, jobs))
            for j, (b, h) in enumerate(chunk):
                zq, zk, zv = arrays[3 * j:3 * j + 3]
                field_q = _smooth_valid(torch.from_numpy(zq), taps) * amp      # [d, T, H, W]
                qf = tile_major(field_q, wl.grid, wl.tile)                     # [N, d] fp32
                kf = qf + 0.5 * tile_major(torch.from_numpy(zk), wl.grid, wl.tile)
                vf = tile_major(torch.from_numpy(zv), wl.grid, wl.tile)
                q[b, h].copy_(qf)
                k[b, h].copy_(kf)
                v[b, h].copy_(vf)
    return q, k, v, head_thresholds(wl)


def small_workload(name: str, heads: int, head_dim: int, block_grid, dtype: str = "bf16",
                   sigma: float = 2.0, threshold: float = 0.9, window=(-1, -1, -1),
                   head_threshold_range=None, seed: int = 0, grid=None) -> Workload:
    """A test-sized workload with the given block grid (tiles 1x8x8), or with the given
    token grid (which may end in partial tiles)."""
    bt, by, bx = block_grid
    g = (bt, 8 * by, 8 * bx) if grid is None else tuple(grid)
    return Workload(name, 1, heads, head_dim, g, dtype, sigma, threshold,
                    head_threshold_range=head_threshold_range, window=tuple(window), seed=seed)
