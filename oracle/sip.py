"""AB-Attention's sampling with inclusion-probability weighting (SIP) -- TEST
INFRASTRUCTURE, part of the oracle (only tests/, smoke() and bench.py's CPU
baseline use it; it shares no code with the HIP library).

AB-Attention page, section "Les trois techniques d'AB-Attention", second item:
a key block enters the sample with a probability proportional to its score, the
most important blocks are always kept, and every kept block is weighted by the
inverse of its inclusion probability (the Horvitz-Thompson estimator), applied as
a logit offset in an ordinary softmax attention.  Readings (the page fixes no
more than that):
  * score: the pooled row softmax p_ij of NABLA's selection ("Methodologie :
    NABLA" on the NABLA summary page), over all key blocks of the row;
  * inclusion probabilities pi_j = min(1, c * p_j) with c > 0 chosen so that
    sum_j pi_j equals the budget k (expected kept blocks per row); blocks whose
    c * p_j reaches 1 are the "always kept" ones.  When k is at least the number
    of blocks with p_j > 0, every such block gets pi_j = 1;
  * sampling: independent draws, block j of row r kept iff u_rj < pi_j, where
    u_rj is the top 24 bits of SplitMix64 output number r * nB + j + 1 of the
    stream seeded with `seed`, scaled by 2^-24;
  * offset: b_j = -ln(pi_j), so a kept block's keys weigh 1 / pi_j in both the
    numerator and the normaliser of the softmax.
All arithmetic is fp64 except the uniforms, which are exact multiples of 2^-24.
"""
from __future__ import annotations

from typing import Optional

import numpy as np

from . import pool, default_scale, csr_from_mask

# SplitMix64 (Steele, Lea and Flood, "Fast splittable pseudorandom number
# generators", OOPSLA 2014): the state advances by the golden gamma and each output
# is the state passed through the variant-13 mix of the murmur3 finaliser.
_GAMMA = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)


def splitmix64(seed: int, counter) -> np.ndarray:
    """Output number `counter` (1-based) of the SplitMix64 stream seeded with `seed`."""
    c = np.asarray(counter, dtype=np.uint64)
    with np.errstate(over="ignore"):
        z = np.uint64(seed & 0xFFFFFFFFFFFFFFFF) + c * _GAMMA
        z = (z ^ (z >> np.uint64(30))) * _M1
        z = (z ^ (z >> np.uint64(27))) * _M2
    return z ^ (z >> np.uint64(31))


def uniforms(seed: int, rows: int, nB: int, row0: int = 0) -> np.ndarray:
    """u[r, j] in [0, 1): top 24 bits of output r * nB + j + 1, times 2^-24."""
    r = np.arange(row0, row0 + rows, dtype=np.uint64)[:, None]
    j = np.arange(nB, dtype=np.uint64)[None, :]
    z = splitmix64(seed, r * np.uint64(nB) + j + np.uint64(1))
    return (z >> np.uint64(40)).astype(np.float64) * 2.0 ** -24


def pooled_probabilities(q, k, heads: int, scale: Optional[float] = None) -> np.ndarray:
    """p [B*H*nB, nB]: softmax over key blocks of the pooled scores Qbar_i . Kbar_j * scale."""
    qb, kb = pool(q), pool(k)                      # [B, H, nB, d] fp64
    d = qb.shape[-1]
    sc = default_scale(d) if scale is None else float(scale)
    s = np.einsum("...id,...jd->...ij", qb, kb) * sc
    s -= s.max(axis=-1, keepdims=True)
    e = np.exp(s)
    p = e / e.sum(axis=-1, keepdims=True)
    return p.reshape(-1, p.shape[-1])


def inclusion_probabilities(p: np.ndarray, budget: float) -> np.ndarray:
    """pi = min(1, c p) per row with sum(pi) = budget (see the module notes).

    For each row, with p sorted descending: try m = 0, 1, ... capped blocks; c is
    (budget - m) / (sum of the rest) and the first m whose next block has
    c * p <= 1 fixes the solution.
    """
    p = np.atleast_2d(np.asarray(p, dtype=np.float64))
    pi = np.zeros_like(p)
    for r in range(p.shape[0]):
        row = p[r]
        npos = int(np.count_nonzero(row > 0))
        if budget >= npos:
            pi[r] = (row > 0).astype(np.float64)
            continue
        ps = np.sort(row)[::-1]
        tail = np.cumsum(ps[::-1])[::-1]           # tail[m] = sum of ps[m:]
        for m in range(npos):
            c = (budget - m) / tail[m]
            if c * ps[m] <= 1.0:
                pi[r] = np.minimum(1.0, c * row)
                break
    return pi


def select_sip(q, k, heads: int, budget: float, seed: int, scale: Optional[float] = None):
    """The sampled block list: (keep [rows, nB] bool, row_ptr, col_idx, bias per entry,
    pi [rows, nB], u [rows, nB])."""
    p = pooled_probabilities(q, k, heads, scale)
    pi = inclusion_probabilities(p, budget)
    u = uniforms(seed, p.shape[0], p.shape[1])
    keep = u < pi
    row_ptr, col_idx = csr_from_mask(keep)
    rows = np.repeat(np.arange(p.shape[0]), np.diff(row_ptr))
    bias = -np.log(pi[rows, col_idx])
    return keep, row_ptr, col_idx, bias, pi, u
