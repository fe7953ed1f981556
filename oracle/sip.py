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
    of blocks with p_j > 0, every such block gets pi_j = 1.  With m blocks capped,
    an uncapped block has pi_j = (k - m) p_j / (mass of the uncapped), which is
    computed from the scores relative to the largest uncapped one so that no
    probability of the row underflows on the way (p_j is never formed);
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


def pooled_scores(q, k, heads: int, scale: Optional[float] = None) -> np.ndarray:
    """S [B*H*nB, nB]: the pooled scores Qbar_i . Kbar_j * scale (fp64), whose row
    softmax is NABLA's p_ij."""
    qb, kb = pool(q), pool(k)                      # [B, H, nB, d] fp64
    d = qb.shape[-1]
    sc = default_scale(d) if scale is None else float(scale)
    s = np.einsum("...id,...jd->...ij", qb, kb) * sc
    return s.reshape(-1, s.shape[-1])


def pooled_probabilities(q, k, heads: int, scale: Optional[float] = None) -> np.ndarray:
    """p [B*H*nB, nB]: the row softmax of pooled_scores."""
    s = pooled_scores(q, k, heads, scale)
    e = np.exp(s - s.max(axis=-1, keepdims=True))
    return e / e.sum(axis=-1, keepdims=True)


def inclusion_probabilities_from_scores(s: np.ndarray, budget: float) -> np.ndarray:
    """pi = min(1, c p) per row with sum(pi) = budget, p = softmax(s) (module notes).

    For each row, with s sorted descending: try m = 0, 1, ... capped blocks.  The
    uncapped ones are those after the m-th; with mR the largest of them and
    E = sum over them of exp(s - mR), an uncapped block gets (budget - m)
    exp(s_j - mR) / E, and the first m for which the largest uncapped block stays
    at or below 1 -- budget - m <= E -- fixes the solution.  Scores of -inf are
    blocks with p = 0: never included.
    """
    s = np.atleast_2d(np.asarray(s, dtype=np.float64))
    pi = np.zeros_like(s)
    for r in range(s.shape[0]):
        row = s[r]
        fin = np.isfinite(row)
        npos = int(fin.sum())
        if budget >= npos:
            pi[r] = fin.astype(np.float64)
            continue
        ss = np.sort(row[fin])[::-1]
        for m in range(npos):
            mR = ss[m]
            E = float(np.exp(ss[m:] - mR).sum())
            K = budget - m
            if K <= E:
                pi[r] = np.where(fin, np.minimum(1.0, K * np.exp(np.where(fin, row, mR) - mR) / E), 0.0)
                break
    return pi


def inclusion_probabilities(p: np.ndarray, budget: float) -> np.ndarray:
    """The same for row probabilities p (p = 0 never included)."""
    p = np.atleast_2d(np.asarray(p, dtype=np.float64))
    with np.errstate(divide="ignore"):
        return inclusion_probabilities_from_scores(np.log(p), budget)


def select_sip(q, k, heads: int, budget: float, seed: int, scale: Optional[float] = None):
    """The sampled block list: (keep [rows, nB] bool, row_ptr, col_idx, bias per entry,
    pi [rows, nB], u [rows, nB])."""
    s = pooled_scores(q, k, heads, scale)
    pi = inclusion_probabilities_from_scores(s, budget)
    u = uniforms(seed, s.shape[0], s.shape[1])
    keep = u < pi
    row_ptr, col_idx = csr_from_mask(keep)
    rows = np.repeat(np.arange(s.shape[0]), np.diff(row_ptr))
    bias = -np.log(pi[rows, col_idx])
    return keep, row_ptr, col_idx, bias, pi, u
