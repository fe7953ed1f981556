"""CPU oracle for dynamic block-sparse video attention -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  It shares no code with the HIP library
and never imports it.

The arithmetic lives in ``oracle.c`` (plain fp64 loops, OpenMP over rows);
this module only marshals NumPy arrays.  What each step computes, and the
readings taken where the NABLA summary page ("NABLA: Neighborhood Adaptive
Block-Level Attention", section "Methodologie : NABLA") is silent, are stated
in ``oracle.c``.

Pinned by ``tests/test_oracle_pins.py`` (closed forms, brute force on tiny
grids, invariants, a hand-derived golden case); no function here is
unpinned.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

TOKENS_PER_BLOCK = 64


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so with gcc (fp64, OpenMP)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + f".tmp{os.getpid()}"
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", "-std=c11",
                               _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
            build()
        lib = ctypes.CDLL(_LIB_PATH)
        P = ctypes.c_void_p
        I = ctypes.c_int64
        D = ctypes.c_double
        lib.oracle_pool.argtypes = [P, I, I, I, P, I, P]
        lib.oracle_select_rows.argtypes = [P, P, I, I, I, I, P, I, D, P, I, I, I, I, I, I, P, P, P]
        lib.oracle_attention_rows.argtypes = [P, P, P, I, I, I, I, P, P, P, P, P, I, D, P, P, P]
        lib.oracle_attention_backward.argtypes = [P, P, P, P, P, I, I, I, I, P, P, P, D, P, P, P]
        for f in (lib.oracle_pool, lib.oracle_select_rows, lib.oracle_attention_rows, lib.oracle_attention_backward):
            f.restype = None
        _lib = lib
    return _lib


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _f32(x) -> np.ndarray:
    """Exact float32 copy of a tensor/array (bf16 and f32 widen exactly)."""
    if hasattr(x, "detach"):
        import torch
        x = x.detach().to("cpu", torch.float32).numpy()
    return np.ascontiguousarray(x, dtype=np.float32)


def default_scale(head_dim: int) -> float:
    return 1.0 / float(np.sqrt(head_dim))


def pool(x, tpb: int = TOKENS_PER_BLOCK, valid: Optional[np.ndarray] = None) -> np.ndarray:
    """Block means: x [..., N, d] -> [..., N/tpb, d] in fp64.  `valid` ([N] bool, the
    same for every head): only those tokens are averaged (padding of partial tiles)."""
    x = _f32(x)
    *lead, n, d = x.shape
    if n % tpb:
        raise ValueError("token count must be a whole number of blocks")
    nblk = int(np.prod(lead, dtype=np.int64)) * (n // tpb)
    vb = _valid(valid, n)
    out = np.empty((nblk, d), dtype=np.float64)
    _load().oracle_pool(_ptr(x), nblk, tpb, d, _ptr(vb), n // tpb, _ptr(out))
    return out.reshape(*lead, n // tpb, d)


def _valid(valid, n):
    if valid is None:
        return None
    vb = np.ascontiguousarray(np.asarray(valid, dtype=bool), dtype=np.uint8)
    if vb.shape != (n,):
        raise ValueError(f"valid must have one entry per token slot ({n})")
    if not vb.reshape(-1, TOKENS_PER_BLOCK).any(axis=1).all():
        raise ValueError("every block needs at least one valid token")
    return vb


def select_rows(qbar: np.ndarray, kbar: np.ndarray, heads: int, block_grid: Sequence[int],
                thresholds, window=(-1, -1, -1), scale: Optional[float] = None,
                rows: Optional[np.ndarray] = None, stats: bool = False):
    """Reduced map, CDF cut and window for the listed rows.

    qbar: pooled [B, H, nB, d], kbar: pooled [B, H, nK, d] (fp64; nK == nB for the
    square map, or the 4-token key blocks of AB-Attention's fine selection, where no
    window applies).  thresholds: scalar or [H].
    Returns ``keep`` [nrows, nK] uint8 (bit 0: CDF rule, bit 1: window) and,
    with ``stats``, the probabilities ``p`` and the exclusive CDF mass ``E``.
    """
    qbar = np.ascontiguousarray(qbar, dtype=np.float64)
    kbar = np.ascontiguousarray(kbar, dtype=np.float64)
    *lead, nB, d = qbar.shape
    nK = kbar.shape[-2]
    bh = int(np.prod(lead, dtype=np.int64))
    nT, nTy, nTx = (int(g) for g in block_grid)
    if nT * nTy * nTx != nB:
        raise ValueError("block grid does not match the number of blocks")
    thr = np.broadcast_to(np.asarray(thresholds, dtype=np.float64), (heads,)).copy()
    if not np.all(thr > 0):
        raise ValueError("thresholds must be > 0")
    if rows is None:
        rows = np.arange(bh * nB, dtype=np.int64)
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    keep = np.zeros((len(rows), nK), dtype=np.uint8)
    p = np.empty((len(rows), nK), dtype=np.float64) if stats else None
    E = np.empty((len(rows), nK), dtype=np.float64) if stats else None
    sc = default_scale(d) if scale is None else float(scale)
    wt, wh, ww = (int(w) for w in window)
    _load().oracle_select_rows(_ptr(qbar), _ptr(kbar), heads, nB, nK, d, _ptr(rows), len(rows), sc,
                               _ptr(thr), nT, nTy, nTx, wt, wh, ww, _ptr(keep), _ptr(p), _ptr(E))
    if stats:
        return keep, p, E
    return keep


def attention_backward(q, k, v, dout, row_ptr, col_idx, scale: Optional[float] = None,
                       tpb: int = TOKENS_PER_BLOCK, out=None, valid=None):
    """Gradients (dq, dk, dv) [B, H, N, d] fp64 of the block-sparse attention for the
    upstream gradient dout, from their definition (see oracle.c).  row_ptr/col_idx: a
    valid CSR (ascending, in-range columns) over rows r = bh * nB + i.  `out`: the
    forward output as stored (e.g. rounded to bf16), used for D = dO . O; None
    recomputes it in fp64.  `valid`: [N] bool, the token slots that are not padding
    (partial tiles); padding slots get zero gradients and no weight as keys."""
    q, k, v, g = _f32(q), _f32(k), _f32(v), _f32(dout)
    o = None if out is None else _f32(out)
    if o is not None and o.shape != q.shape:
        raise ValueError("out must have the shape of q")
    *lead, n, d = q.shape
    BH = int(np.prod(lead)) if lead else 1
    nB = n // tpb
    rp = np.ascontiguousarray(row_ptr, dtype=np.int64)
    ci = np.ascontiguousarray(col_idx, dtype=np.int32)
    dq = np.empty(q.shape, dtype=np.float64)
    dk = np.empty(q.shape, dtype=np.float64)
    dv = np.empty(q.shape, dtype=np.float64)
    sc = default_scale(d) if scale is None else float(scale)
    vb = None if valid is None else np.ascontiguousarray(np.asarray(valid, dtype=bool), dtype=np.uint8)
    if vb is not None and (vb.shape != (n,) or not vb.reshape(-1, tpb).any(axis=1).all()):
        raise ValueError("valid needs one entry per token slot and a token in every block")
    _load().oracle_attention_backward(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(o), BH, nB, tpb, d, _ptr(rp), _ptr(ci),
                                      _ptr(vb), sc, _ptr(dq), _ptr(dk), _ptr(dv))
    return dq, dk, dv


def block_grid(grid: Sequence[int], tile: Sequence[int]):
    """Tiles along t, y, x: ceil(grid / tile) (a last partial tile counts as a tile)."""
    return tuple(-(-int(g) // int(s)) for g, s in zip(grid, tile))


def tile_order(grid: Sequence[int], tile: Sequence[int]) -> np.ndarray:
    """perm[i] = raster index of the token at tile-major position i, or -1 for padding.

    NABLA summary page, section "Methodologie : NABLA", item "Fractal Flattening":
    the tokens of each spatial patch are made contiguous, whatever the global size of
    the video.  Raster token (t, y, x) sits at (t * H + y) * W + x; tile-major position
    i belongs to block b = i // V (V = tile volume), b = (bt * nTy + by) * nTx + bx over
    the ceil(grid / tile) tiles, and is the (i mod V)-th slot of that tile in row-major
    order.  A slot whose coordinates fall beyond the grid (a partial tile at the far
    edge of t, y or x) is padding.
    """
    T, H, W = (int(g) for g in grid)
    tt, th, tw = (int(s) for s in tile)
    vol = tt * th * tw
    nT, nTy, nTx = block_grid(grid, tile)
    i = np.arange(nT * nTy * nTx * vol, dtype=np.int64)
    b, u = i // vol, i % vol
    bt, by, bx = b // (nTy * nTx), (b // nTx) % nTy, b % nTx
    ut, uy, ux = u // (th * tw), (u // tw) % th, u % tw
    t, y, x = bt * tt + ut, by * th + uy, bx * tw + ux
    ok = (t < T) & (y < H) & (x < W)
    return np.where(ok, (t * H + y) * W + x, -1)


def token_valid(grid: Sequence[int], tile: Sequence[int]) -> np.ndarray:
    """[nB * V] bool: which tile-major slots hold a token of the grid (not padding)."""
    return tile_order(grid, tile) >= 0


def to_tiles(x, grid, tile) -> np.ndarray:
    """Raster-ordered [..., N, d] -> tile-major [..., nB * V, d] (same dtype, exact; padding
    slots are zero)."""
    a = x.numpy() if hasattr(x, "numpy") else np.asarray(x)
    perm = tile_order(grid, tile)
    out = np.zeros(a.shape[:-2] + (len(perm), a.shape[-1]), dtype=a.dtype)
    ok = perm >= 0
    out[..., ok, :] = a[..., perm[ok], :]
    return out


def from_tiles(x, grid, tile) -> np.ndarray:
    """Tile-major [..., nB * V, d] -> raster order [..., N, d] (the inverse of to_tiles;
    padding slots are dropped)."""
    a = x.numpy() if hasattr(x, "numpy") else np.asarray(x)
    perm = tile_order(grid, tile)
    T, H, W = (int(g) for g in grid)
    out = np.empty(a.shape[:-2] + (T * H * W, a.shape[-1]), dtype=a.dtype)
    ok = perm >= 0
    out[..., perm[ok], :] = a[..., ok, :]
    return out


def csr_from_mask(mask: np.ndarray):
    """Dense boolean block mask [rows, nB] -> (row_ptr int64 [rows+1], col_idx int32), ascending columns."""
    mask = np.asarray(mask).astype(bool)
    counts = mask.sum(axis=1)
    row_ptr = np.zeros(mask.shape[0] + 1, dtype=np.int64)
    np.cumsum(counts, out=row_ptr[1:])
    col_idx = np.nonzero(mask)[1].astype(np.int32)
    return row_ptr, col_idx


def select(q, k, heads: int, block_grid, thresholds, window=(-1, -1, -1), scale=None, valid=None):
    """Full selection for every row: returns (mask bool [B*H*nB, nB], row_ptr, col_idx).
    `valid`: the token slots that are not padding (partial tiles), as in pool()."""
    qbar = pool(q, valid=valid)
    kbar = pool(k, valid=valid)
    keep = select_rows(qbar, kbar, heads, block_grid, thresholds, window, scale)
    mask = keep != 0
    row_ptr, col_idx = csr_from_mask(mask)
    return mask, row_ptr, col_idx


def attention_rows(q, k, v, row_ptr, col_idx, rows, scale: Optional[float] = None,
                   tpb: int = TOKENS_PER_BLOCK, weights: bool = False, bias=None, valid=None,
                   key_tokens: Optional[int] = None):
    """Exact attention of every token of the listed query-block rows over its kept tiles.

    q, k, v: [B, H, N, d]; row_ptr/col_idx: CSR over rows r = bh * nB + i.
    Returns out [nrows, tpb, d] fp64 and lse [nrows, tpb] (natural log), plus
    the per-token weight sums with ``weights``.  ``bias``: optional logit offset per
    col_idx entry, added to the scaled logits of all keys of that block.  ``valid``:
    [N] bool, the token slots that are not padding (partial tiles); padding keys get no
    weight and padding queries O = 0, LSE = -inf.  ``key_tokens``: tokens per key block
    (default tpb; 4 for AB-Attention's 4-token key blocks, col_idx then indexing them).
    """
    q, k, v = _f32(q), _f32(k), _f32(v)
    *lead, n, d = q.shape
    nB = n // tpb
    b = None if bias is None else np.ascontiguousarray(bias, dtype=np.float64)
    if b is not None and b.shape != np.shape(col_idx):
        raise ValueError("bias needs one value per col_idx entry")
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    rp = np.ascontiguousarray(row_ptr, dtype=np.int64)
    ci = np.ascontiguousarray(col_idx, dtype=np.int32)
    out = np.empty((len(rows), tpb, d), dtype=np.float64)
    lse = np.empty((len(rows), tpb), dtype=np.float64)
    ws = np.empty((len(rows), tpb), dtype=np.float64) if weights else None
    sc = default_scale(d) if scale is None else float(scale)
    vb = _valid(valid, n)
    tk = tpb if key_tokens is None else int(key_tokens)
    if n % tk or (vb is not None and tk != tpb):
        raise ValueError("key blocks must tile the tokens (and padding needs whole tiles as key blocks)")
    _load().oracle_attention_rows(_ptr(q), _ptr(k), _ptr(v), nB, tpb, tk, d, _ptr(rp), _ptr(ci), _ptr(b), _ptr(vb),
                                  _ptr(rows), len(rows), sc, _ptr(out), _ptr(lse), _ptr(ws))
    if weights:
        return out, lse, ws
    return out, lse


# ---------------------------------------------------------------- AB-Attention's fine selection
KEY_BLOCK_4 = 4


def select_fine(q, k, heads: int, thresholds, key_tokens: int = KEY_BLOCK_4, scale=None, stats: bool = False):
    """AB-Attention page, section "Les trois techniques d'AB-Attention", third technique:
    key blocks of `key_tokens` (4) tokens, selected per 64-token query block.  Reading:
    the query blocks are NABLA's 64-token means, the key blocks the means of `key_tokens`
    consecutive tile-major tokens (half a row of an 8 x 8 tile); each row is the softmax
    of the pooled scores over all key blocks of the head, cut by NABLA's CDF rule.
    Returns (keep bool [B*H*nB, nK], row_ptr, col_idx) -- col_idx indexes key blocks --
    plus (p, E) with ``stats``."""
    qbar = pool(q)
    kbar = pool(k, tpb=key_tokens)
    *lead, nB, _ = qbar.shape
    r = select_rows(qbar, kbar, heads, (1, 1, nB), thresholds, (-1, -1, -1), scale, stats=stats)
    keep = (r[0] if stats else r) != 0
    row_ptr, col_idx = csr_from_mask(keep)
    if stats:
        return keep, row_ptr, col_idx, r[1], r[2]
    return keep, row_ptr, col_idx
