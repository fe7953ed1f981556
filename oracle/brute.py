"""Brute-force NumPy checks for the oracle -- TEST INFRASTRUCTURE.

Independent re-derivations used only to pin ``oracle.c`` on tiny inputs.
Each one reaches the same result by a different route than the oracle:

* ``cdf_keep_pairwise``: the CDF rule of the NABLA summary page (section
  "Methodologie : NABLA", "Seuil CDF") evaluated without sorting: for each
  block j, the mass of every block ordered before it (higher probability, or
  equal probability and lower index) is summed directly, O(nB^2).
* ``token_mask_attention``: the "Expansion" step taken literally -- the block
  mask is expanded to a token-level N x N mask, disallowed logits are set to
  -inf and an ordinary dense softmax runs over the whole key axis.
* ``dense_attention``: textbook softmax attention, used for thr >= 1.
* ``raster_block_mask_attention``: the same literal expansion on a raster-ordered
  grid that need not be a whole number of tiles: every token's block is found
  from its own (t, y, x) coordinates, with no tile-major reordering or padding.
* ``window_count``: the number of blocks in a clipped box window, as a product
  of per-axis interval lengths.
"""
from __future__ import annotations

import numpy as np


def cdf_keep_pairwise(p: np.ndarray, thr: float) -> np.ndarray:
    """Keep mask of one probability row by direct evaluation of E(j) < thr."""
    p = np.asarray(p, dtype=np.float64)
    n = p.shape[0]
    if thr >= 1.0:
        return np.ones(n, dtype=bool)
    idx = np.arange(n)
    before = (p[None, :] > p[:, None]) | ((p[None, :] == p[:, None]) & (idx[None, :] < idx[:, None]))
    E = np.where(before, p[None, :], 0.0).sum(axis=1)
    return E < thr


def dense_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float):
    """softmax(q k^T * scale) v over the whole key axis (fp64), plus the log-sum-exp."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    s = (q @ k.T) * scale
    m = s.max(axis=-1, keepdims=True)
    e = np.exp(s - m)
    z = e.sum(axis=-1, keepdims=True)
    return (e / z) @ v, (m + np.log(z))[..., 0]


def token_mask_attention(q, k, v, block_mask: np.ndarray, scale: float, tpb: int = 64, key_tokens=None):
    """Masked dense attention with the block mask expanded to tokens (fp64).

    q, k, v: [N, d] for one head; block_mask: [nB, nK] bool, query blocks of tpb
    tokens, key blocks of key_tokens (default tpb) tokens.
    Rows with no allowed key give O = 0 and LSE = -inf.
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    tk = tpb if key_tokens is None else key_tokens
    tok = np.kron(np.asarray(block_mask, dtype=np.int8), np.ones((tpb, tk), dtype=np.int8)).astype(bool)
    s = np.where(tok, (q @ k.T) * scale, -np.inf)
    out = np.zeros((q.shape[0], v.shape[1]))
    lse = np.full(q.shape[0], -np.inf)
    ok = tok.any(axis=1)
    m = s[ok].max(axis=1, keepdims=True)
    e = np.exp(s[ok] - m)
    z = e.sum(axis=1, keepdims=True)
    out[ok] = (e / z) @ v
    lse[ok] = (m + np.log(z))[:, 0]
    return out, lse


def window_count(i: int, block_grid, window) -> int:
    """Blocks inside the clipped box window around block i."""
    nT, nTy, nTx = block_grid
    t, y, x = i // (nTy * nTx), (i // nTx) % nTy, i % nTx
    n = 1
    for c, r, size in ((t, window[0], nT), (y, window[1], nTy), (x, window[2], nTx)):
        n *= min(size - 1, c + r) - max(0, c - r) + 1
    return n


def raster_block_of(grid, tile) -> np.ndarray:
    """Block index of every raster token (t, y, x): (t // tt, y // th, x // tw) over the
    ceil(grid / tile) blocks."""
    T, H, W = grid
    tt, th, tw = tile
    nTy, nTx = -(-H // th), -(-W // tw)
    t, y, x = np.meshgrid(np.arange(T), np.arange(H), np.arange(W), indexing="ij")
    return (((t // tt) * nTy + (y // th)) * nTx + (x // tw)).reshape(-1)


def raster_block_mask_attention(q, k, v, grid, tile, block_mask: np.ndarray, scale: float):
    """Masked dense attention of raster-ordered tokens [N, d] (one head): token n may
    attend to token m iff block_mask[block(n), block(m)], blocks taken from the tokens'
    grid coordinates (fp64).  Returns out [N, d] and lse [N]."""
    blk = raster_block_of(grid, tile)
    allowed = np.asarray(block_mask, dtype=bool)[blk[:, None], blk[None, :]]
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    s = np.where(allowed, (q @ k.T) * scale, -np.inf)
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    z = e.sum(axis=1, keepdims=True)
    return (e / z) @ v, (m + np.log(z))[:, 0]
