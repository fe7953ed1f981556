"""AB-Attention's intra-block clustering selector (IBCS) -- TEST INFRASTRUCTURE,
part of the oracle (only tests/, smoke() and bench.py's CPU baseline use it; no
code shared with the HIP library).

AB-Attention page, section "Les trois techniques d'AB-Attention", first item:
queries are cut into blocks of 128 tokens; within each block they are grouped
into 8 clusters, each with a centroid and a weight equal to its share of the
block's queries; a key block's score is the weighted attention of the centroids
on its mean-pooled keys; the clusters serve the estimate only (the attention
itself keeps the token order).  Readings (the page names no algorithm):
  * a 128-token query block is a pair of 64-token blocks (2p, 2p+1) in tile-major
    order (an odd last block stands alone, 64 tokens); both blocks get the pair's
    score row and are cut with it;
  * clustering: Lloyd's k-means, K = 8, ITERS = 4 rounds of (assign each query to
    the nearest centroid by squared Euclidean distance, ties to the lower cluster;
    move each centroid to the mean of its queries, an empty cluster keeping its
    centroid), started from the queries at positions n*c/8 (c = 0..7) of the
    block; the weights are the shares of the last assignment;
  * keys: NABLA's 64-token mean-pooled K (its "Sous-echantillonnage");
  * score: p~_j = sum_c w_c softmax_j(mu_c . Kbar_j * scale) over all key blocks;
  * the cut: NABLA's CDF rule on p~ (descending order, ties to the lower index,
    keep while the mass before a block is below thr; thr >= 1 keeps all).
All in fp64.  `kmeans` also reports, for the block, the smallest relative gap
between a query's nearest and second-nearest centroid over all rounds, which
says how close an assignment came to a tie.
"""
from __future__ import annotations

from typing import Optional

import numpy as np

from . import pool, default_scale, csr_from_mask

K_CLUSTERS = 8
ITERS = 4
QBLOCK = 128


def kmeans(x: np.ndarray, k: int = K_CLUSTERS, iters: int = ITERS):
    """x [n, d] -> (centroids [k, d], weights [k], smallest relative assignment gap)."""
    x = np.asarray(x, dtype=np.float64)
    n = x.shape[0]
    mu = x[[(n * c) // k for c in range(k)]].copy()
    gap = np.inf
    a = np.zeros(n, dtype=np.int64)
    for _ in range(iters):
        d2 = ((x[:, None, :] - mu[None, :, :]) ** 2).sum(axis=-1)        # [n, k]
        a = np.argmin(d2, axis=1)                                         # ties -> lower index
        srt = np.sort(d2, axis=1)
        rel = (srt[:, 1] - srt[:, 0]) / np.maximum(srt[:, 1], 1e-300)
        gap = min(gap, float(rel.min()))
        for c in range(k):
            m = a == c
            if m.any():
                mu[c] = x[m].mean(axis=0)
    w = np.bincount(a, minlength=k).astype(np.float64) / n
    return mu, w, gap


def mixture_scores(q, k, heads: int, scale: Optional[float] = None, iters: int = ITERS):
    """p~ [B*H*nB, nB] (the pair's row for both of its blocks) and the smallest
    assignment gap per pair [B*H, ceil(nB/2)].  `iters`: k-means rounds (the reading
    is ITERS; other counts serve tests that show the round count matters)."""
    q = np.asarray(q, dtype=np.float64)
    kb = pool(k)                                   # [B, H, nB, d] fp64
    *lead, N, d = q.shape
    nB = kb.shape[-2]
    sc = default_scale(d) if scale is None else float(scale)
    qf = q.reshape(-1, N, d)
    kf = kb.reshape(-1, nB, d)
    BH = qf.shape[0]
    npairs = (nB + 1) // 2
    pt = np.empty((BH, nB, nB))
    gaps = np.empty((BH, npairs))
    for bh in range(BH):
        for p in range(npairs):
            t0, t1 = 128 * p, min(128 * p + 128, N)
            mu, w, gaps[bh, p] = kmeans(qf[bh, t0:t1], iters=iters)
            s = mu @ kf[bh].T * sc                 # [8, nB]
            e = np.exp(s - s.max(axis=1, keepdims=True))
            row = (w[:, None] * e / e.sum(axis=1, keepdims=True)).sum(axis=0)
            pt[bh, 2 * p] = row
            if 2 * p + 1 < nB:
                pt[bh, 2 * p + 1] = row
    return pt.reshape(BH * nB, nB), gaps


def cdf_keep(p: np.ndarray, thr: float) -> np.ndarray:
    """NABLA's CDF rule on rows of probabilities (sum 1): order by p descending, ties to
    the lower index, keep a block while the mass strictly before it is below thr."""
    p = np.atleast_2d(np.asarray(p, dtype=np.float64))
    if thr >= 1.0:
        return np.ones(p.shape, dtype=bool)
    keep = np.zeros(p.shape, dtype=bool)
    for r in range(p.shape[0]):
        order = np.argsort(-p[r], kind="stable")
        before = np.concatenate([[0.0], np.cumsum(p[r][order])[:-1]])
        keep[r, order] = before < thr
    return keep


def select_ibcs(q, k, heads: int, thr: float, scale: Optional[float] = None, iters: int = ITERS):
    """(keep [rows, nB], row_ptr, col_idx, p~ [rows, nB], gaps [B*H, pairs])."""
    pt, gaps = mixture_scores(q, k, heads, scale, iters)
    keep = cdf_keep(pt, thr)
    row_ptr, col_idx = csr_from_mask(keep)
    return keep, row_ptr, col_idx, pt, gaps
