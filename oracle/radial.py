"""DynamicRad's radial window as a block mask -- TEST INFRASTRUCTURE, part of the
oracle (only tests/, smoke() and bench.py's CPU baseline use it; no code shared
with the HIP library).

DynamicRad page, section "Methodologie : DynamicRad", items A (a shared candidate
set built on a radial locality prior: attention energy decays with spatial and
temporal distance) and B (a decay factor gamma that sets the width of the local
window as a function of temporal distance, and a long-range factor lambda that
sets how often distant frames are sampled).  The page gives no formula; the
reading used here, in block (tile) coordinates:
  * width w(dt) = r0 * gamma^dt for frame distance dt, formed by dt successive
    fp64 multiplications of r0 by gamma (r0, gamma given as fp32);
  * radius R(dt) = floor(w(dt)) while w(dt) >= 1; a frame with w(dt) < 1 is
    skipped, except that when lambda >= 1 and dt is a multiple of lambda it keeps
    the co-located block (R = 0); the own frame always has R(0) = max(floor(r0), 0);
  * key block j is kept for query block i iff the spatial Chebyshev distance
    max(|dy|, |dx|) <= R(|dt|) (no wrap, clipped at the grid edges).
"""
from __future__ import annotations

import math

import numpy as np


def radii(n_frames: int, r0: float, gamma: float, lam: int) -> np.ndarray:
    """R(dt) for dt = 0 .. n_frames-1 (int64; -1 = frame skipped)."""
    r0d, gd = float(np.float32(r0)), float(np.float32(gamma))
    out = np.empty(n_frames, dtype=np.int64)
    w = r0d
    for dt in range(n_frames):
        if dt > 0:
            w = w * gd
        if dt == 0:
            out[dt] = max(int(math.floor(min(w, 1e6))), 0)
        elif w >= 1.0:
            out[dt] = int(math.floor(min(w, 1e6)))
        elif lam >= 1 and dt % lam == 0:
            out[dt] = 0
        else:
            out[dt] = -1
    return out


def radial_mask(block_grid, r0: float, gamma: float, lam: int) -> np.ndarray:
    """keep [nB, nB] bool for one head (the same for every head)."""
    nT, nTy, nTx = (int(x) for x in block_grid)
    R = radii(nT, r0, gamma, lam)
    i = np.arange(nT * nTy * nTx)
    t, y, x = i // (nTy * nTx), (i // nTx) % nTy, i % nTx
    dt = np.abs(t[:, None] - t[None, :])
    ds = np.maximum(np.abs(y[:, None] - y[None, :]), np.abs(x[:, None] - x[None, :]))
    return ds <= R[dt]
