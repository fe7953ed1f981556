"""Pins of the CPU oracle against things other than itself (CPU only).

Closed forms, a hand-derived worked example, brute force on tiny grids and
invariants, chosen so that a dropped term, a wrong sign, index or scale, or a
transposed operand in ``oracle.c`` fails at least one of them.
"""
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import brute

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "dyadic_cdf.txt")


def _rand(shape, seed, scale=1.0):
    return (np.random.default_rng(seed).standard_normal(shape) * scale).astype(np.float32)


# ---------------------------------------------------------------- pooling

def test_pool_constant_and_ramp():
    # constant tokens pool to the constant; a ramp over the 64 tokens pools to its midpoint
    x = np.zeros((2, 128, 4), np.float32)
    x[:, :64, 0] = 3.25
    x[:, 64:, 1] = np.arange(64, dtype=np.float32)
    x[:, :, 2] = np.arange(128, dtype=np.float32)[None, :] * 0.5
    xb = oracle.pool(x)
    assert xb.shape == (2, 2, 4)
    assert np.all(xb[:, 0, 0] == 3.25) and np.all(xb[:, 1, 0] == 0)
    assert np.all(xb[:, 1, 1] == 31.5) and np.all(xb[:, 0, 1] == 0)
    assert np.allclose(xb[:, 0, 2], 0.5 * 31.5) and np.allclose(xb[:, 1, 2], 0.5 * 95.5)


def test_pool_matches_reshape_mean():
    x = _rand((3, 5 * 64, 16), 1)
    ref = x.astype(np.float64).reshape(3, 5, 64, 16).mean(axis=2)
    assert np.allclose(oracle.pool(x), ref, rtol=0, atol=1e-12)


# ---------------------------------------------------------------- CDF rule

def _golden_cases():
    cases = []
    for line in open(GOLDEN):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        parts = line.split()
        ns = [int(t) for t in parts[1:5]]
        cases.append((parts[0], ns, float(parts[5]), [int(t) for t in parts[6].split(",")]))
    return cases


@pytest.mark.parametrize("case", _golden_cases(), ids=lambda c: f"{c[0]}-{c[2]}")
def test_golden_dyadic(case):
    _, ns, thr, kept = case
    d = 64
    q = np.zeros((1, 1, 4 * 64, d), np.float32)
    k = np.zeros((1, 1, 4 * 64, d), np.float32)
    q[..., 0] = 8.0
    for j, n in enumerate(ns):
        k[0, 0, 64 * j:64 * (j + 1), 0] = math.log(2.0) * n
    keep, p, E = oracle.select_rows(oracle.pool(q), oracle.pool(k), 1, (1, 1, 4), thr, stats=True)
    expect_p = np.array([2.0 ** n for n in ns]) / sum(2.0 ** n for n in ns)
    assert np.allclose(p[0], expect_p, rtol=1e-6)
    got = sorted(np.nonzero(keep[0] & 1)[0].tolist())
    assert got == kept


@pytest.mark.parametrize("nB,thr", [(16, 0.9), (16, 0.5), (7, 0.3), (480, 0.905), (3840, 0.7001), (5, 1.0), (33, 0.999)])
def test_uniform_scores_keep_ceil(nB, thr):
    # Q = 0 makes every reduced score 0, so p = 1/nB and E = k/nB in index order:
    # the rule keeps the ceil(thr * nB) lowest indices.  Cases where thr * nB is a whole number
    # but 1/nB is not dyadic are left out: there E == thr up to the last bit of the running sum.
    d = 8
    q = np.zeros((1, 1, nB * 64, d), np.float32)
    k = _rand((1, 1, nB * 64, d), 2)
    keep = oracle.select_rows(oracle.pool(q), oracle.pool(k), 1, (1, 1, nB), thr)
    expect = min(nB, math.ceil(thr * nB - 1e-12))
    if thr >= 1:
        expect = nB
    kept = np.nonzero(keep[0] & 1)[0]
    assert len(kept) == expect
    assert np.array_equal(kept, np.arange(expect))


def test_one_hot_and_small_threshold():
    # one key block far above the rest: p_max ~ 1 > thr, so only it is kept;
    # a tiny threshold keeps only the argmax whatever the spread
    nB, d = 12, 16
    q = np.zeros((1, 1, nB * 64, d), np.float32)
    q[..., 0] = 1.0
    k = np.zeros((1, 1, nB * 64, d), np.float32)
    k[0, 0, 5 * 64:6 * 64, 0] = 200.0
    keep = oracle.select_rows(oracle.pool(q), oracle.pool(k), 1, (1, 1, nB), 0.9)
    assert np.nonzero(keep[0])[0].tolist() == [5]
    kr = _rand((1, 1, nB * 64, d), 3)
    qr = _rand((1, 1, nB * 64, d), 4)
    qb, kb = oracle.pool(qr), oracle.pool(kr)
    keep, p, _ = oracle.select_rows(qb, kb, 1, (1, 1, nB), 1e-9, stats=True)
    for r in range(nB):
        assert np.nonzero(keep[r])[0].tolist() == [int(np.argmax(p[r]))]


def test_two_block_sigmoid_closed_form():
    # two key blocks with reduced scores c0, c1: p0 = 1 / (1 + exp(c1 - c0)); checks the 1/sqrt(d) scale
    d = 16
    q = np.zeros((1, 1, 128, d), np.float32)
    k = np.zeros((1, 1, 128, d), np.float32)
    q[..., 3] = 2.0
    k[0, 0, :64, 3] = 1.5
    k[0, 0, 64:, 3] = -0.5
    _, p, _ = oracle.select_rows(oracle.pool(q), oracle.pool(k), 1, (1, 1, 2), 0.5, stats=True)
    c0, c1 = 2.0 * 1.5 / 4.0, 2.0 * -0.5 / 4.0
    assert abs(p[0, 0] - 1.0 / (1.0 + math.exp(c1 - c0))) < 1e-14
    # an explicit scale overrides the default
    _, p2, _ = oracle.select_rows(oracle.pool(q), oracle.pool(k), 1, (1, 1, 2), 0.5, scale=1.0, stats=True)
    assert abs(p2[0, 0] - 1.0 / (1.0 + math.exp(-4.0))) < 1e-14


@pytest.mark.parametrize("seed", range(6))
def test_cdf_matches_pairwise_bruteforce(seed):
    # random tiny heads; the sorted walk of the oracle must equal the sort-free O(n^2) definition,
    # and its probabilities must equal a NumPy softmax of NumPy matmul scores of the pooled vectors
    rng = np.random.default_rng(100 + seed)
    H, nB, d = 3, int(rng.integers(2, 40)), 16
    amp = float(rng.choice([0.3, 3.0, 30.0]))
    q = _rand((1, H, nB * 64, d), seed, amp)
    k = _rand((1, H, nB * 64, d), seed + 50, amp)
    thr = rng.uniform(0.05, 0.99, size=H)
    qb, kb = oracle.pool(q), oracle.pool(k)
    keep, p, E = oracle.select_rows(qb, kb, H, (1, 1, nB), thr, stats=True)
    for h in range(H):
        s = (qb[0, h] @ kb[0, h].T) / math.sqrt(d)
        ref_p = np.exp(s - s.max(axis=1, keepdims=True))
        ref_p /= ref_p.sum(axis=1, keepdims=True)
        assert np.allclose(p[h * nB:(h + 1) * nB], ref_p, rtol=1e-12, atol=1e-300)
        for i in range(nB):
            r = h * nB + i
            assert np.array_equal(keep[r] & 1, brute.cdf_keep_pairwise(p[r], thr[h]).astype(np.uint8))


@pytest.mark.parametrize("seed", range(4))
def test_kept_mass_and_minimality(seed):
    H, nB, d = 2, 64, 32
    q = _rand((1, H, nB * 64, d), 10 + seed, 2.0)
    k = _rand((1, H, nB * 64, d), 20 + seed, 2.0)
    thr = [0.3, 0.85]
    keep, p, _ = oracle.select_rows(oracle.pool(q), oracle.pool(k), H, (1, 1, nB), thr, stats=True)
    for r in range(H * nB):
        t = thr[r // nB]
        kp = p[r][(keep[r] & 1) != 0]
        assert kp.sum() >= t - 1e-12                  # enough mass
        assert kp.sum() - kp.min() < t + 1e-12        # dropping the smallest kept block falls short
        # every dropped block is no more probable than every kept one
        dp = p[r][(keep[r] & 1) == 0]
        if dp.size:
            assert dp.max() <= kp.min()


def test_threshold_one_keeps_underflowed_blocks():
    # thr >= 1 keeps everything, even blocks whose probability underflows to 0
    nB, d = 6, 4
    q = np.zeros((1, 1, nB * 64, d), np.float32)
    q[..., 0] = 1.0
    k = np.zeros((1, 1, nB * 64, d), np.float32)
    k[0, 0, :64, 0] = 3000.0
    keep, p, _ = oracle.select_rows(oracle.pool(q), oracle.pool(k), 1, (1, 1, nB), 1.0, stats=True)
    assert np.all(p[0, 1:] == 0.0)
    assert np.all(keep == 1)
    keep2 = oracle.select_rows(oracle.pool(q), oracle.pool(k), 1, (1, 1, nB), 1.5)
    assert np.all(keep2 == 1)


def test_invalid_threshold_rejected():
    qb = np.zeros((1, 1, 2, 4))
    with pytest.raises(ValueError):
        oracle.select_rows(qb, qb, 1, (1, 1, 2), 0.0)
    with pytest.raises(ValueError):
        oracle.select_rows(qb, qb, 1, (1, 1, 2), float("nan"))


def test_key_block_permutation_permutes_mask():
    # relabelling key blocks relabels the mask columns (random data: no exact ties)
    H, nB, d = 1, 24, 16
    q = _rand((1, H, nB * 64, d), 7, 3.0)
    k = _rand((1, H, nB * 64, d), 8, 3.0)
    perm = np.random.default_rng(9).permutation(nB)
    kp = k.reshape(1, H, nB, 64, d)[:, :, perm].reshape(1, H, nB * 64, d)
    qb = oracle.pool(q)
    a = oracle.select_rows(qb, oracle.pool(k), H, (1, 1, nB), 0.6)
    b = oracle.select_rows(qb, oracle.pool(kp), H, (1, 1, nB), 0.6)
    assert np.array_equal(a[:, perm], b)


# ---------------------------------------------------------------- window

@pytest.mark.parametrize("grid,win", [((3, 4, 5), (1, 1, 1)), ((4, 6, 10), (1, 1, 1)), ((2, 3, 3), (0, 1, 2)),
                                      ((5, 2, 7), (2, 0, 1))])
def test_window_counts(grid, win):
    nB = int(np.prod(grid))
    d = 4
    q = np.zeros((1, 1, nB * 64, d), np.float32)
    k = np.zeros((1, 1, nB * 64, d), np.float32)
    keep = oracle.select_rows(oracle.pool(q), oracle.pool(k), 1, grid, 1e-6, window=win)
    nT, nTy, nTx = grid
    for i in range(nB):
        wmask = (keep[i] & 2) != 0
        assert wmask.sum() == brute.window_count(i, grid, win)
        assert wmask[i]
        t, y, x = i // (nTy * nTx), (i // nTx) % nTy, i % nTx
        for j in np.nonzero(wmask)[0]:
            tj, yj, xj = j // (nTy * nTx), (j // nTx) % nTy, j % nTx
            assert abs(tj - t) <= win[0] and abs(yj - y) <= win[1] and abs(xj - x) <= win[2]
    if grid == (4, 6, 10) and win == (1, 1, 1):
        interior = (1 * 6 + 2) * 10 + 3
        assert (keep[interior] & 2).astype(bool).sum() == 27
        assert (keep[0] & 2).astype(bool).sum() == 8


# ---------------------------------------------------------------- attention

def _full_csr(rows, nB):
    return oracle.csr_from_mask(np.ones((rows, nB), bool))


@pytest.mark.parametrize("d", [16, 64])
def test_threshold_one_equals_dense_attention(d):
    H, nB = 2, 5
    q = _rand((1, H, nB * 64, d), 31, 1.5)
    k = _rand((1, H, nB * 64, d), 32, 1.5)
    v = _rand((1, H, nB * 64, d), 33)
    mask, rp, ci = oracle.select(q, k, H, (1, 1, nB), 1.0)
    assert mask.all()
    out, lse = oracle.attention_rows(q, k, v, rp, ci, np.arange(H * nB))
    sc = 1.0 / math.sqrt(d)
    for h in range(H):
        ref, ref_lse = brute.dense_attention(q[0, h], k[0, h], v[0, h], sc)
        assert np.abs(out[h * nB:(h + 1) * nB].reshape(-1, d) - ref).max() < 1e-12
        assert np.abs(lse[h * nB:(h + 1) * nB].reshape(-1) - ref_lse).max() < 1e-12
        # and the library routine agrees (torch's fp64 scaled-dot-product attention)
        t = torch.nn.functional.scaled_dot_product_attention(
            *(torch.from_numpy(x[0, h].astype(np.float64))[None] for x in (q, k, v)))
        assert np.abs(out[h * nB:(h + 1) * nB].reshape(-1, d) - t[0].numpy()).max() < 1e-12


@pytest.mark.parametrize("seed", range(3))
def test_tile_walk_matches_token_mask_bruteforce(seed):
    rng = np.random.default_rng(seed)
    H, nB, d = 2, 6, 32
    q = _rand((1, H, nB * 64, d), 40 + seed, 2.0)
    k = _rand((1, H, nB * 64, d), 50 + seed, 2.0)
    v = _rand((1, H, nB * 64, d), 60 + seed)
    mask = rng.random((H * nB, nB)) < 0.45
    mask[3] = False                                   # one empty row
    rp, ci = oracle.csr_from_mask(mask)
    out, lse, ws = oracle.attention_rows(q, k, v, rp, ci, np.arange(H * nB), weights=True)
    sc = 1.0 / math.sqrt(d)
    for h in range(H):
        ref, ref_lse = brute.token_mask_attention(q[0, h], k[0, h], v[0, h], mask[h * nB:(h + 1) * nB], sc)
        got = out[h * nB:(h + 1) * nB].reshape(-1, d)
        assert np.abs(got - ref).max() < 1e-12
        gl = lse[h * nB:(h + 1) * nB].reshape(-1)
        assert np.array_equal(np.isinf(gl), np.isinf(ref_lse))
        fin = np.isfinite(ref_lse)
        assert np.abs(gl[fin] - ref_lse[fin]).max() < 1e-12
    nonempty = mask.any(axis=1)
    assert np.abs(ws[nonempty] - 1.0).max() < 1e-12        # each row's weights sum to 1
    assert np.all(out[3] == 0) and np.all(np.isneginf(lse[3]))


def test_constant_values_give_constant_output_and_order_invariance():
    H, nB, d = 1, 8, 16
    q = _rand((1, H, nB * 64, d), 70, 3.0)
    k = _rand((1, H, nB * 64, d), 71, 3.0)
    v = np.broadcast_to(np.linspace(-2, 2, d, dtype=np.float32), (1, H, nB * 64, d)).copy()
    mask = np.random.default_rng(72).random((nB, nB)) < 0.5
    mask[:, 0] = True
    rp, ci = oracle.csr_from_mask(mask)
    out, _ = oracle.attention_rows(q, k, v, rp, ci, np.arange(nB))
    assert np.abs(out - v[0, 0, 0]).max() < 1e-12
    # the order in which a row's tiles are walked does not change the result
    v2 = _rand((1, H, nB * 64, d), 73)
    a, la = oracle.attention_rows(q, k, v2, rp, ci, np.arange(nB))
    ci_rev = ci.copy()
    for r in range(nB):
        ci_rev[rp[r]:rp[r + 1]] = ci[rp[r]:rp[r + 1]][::-1]
    b, lb = oracle.attention_rows(q, k, v2, rp, ci_rev, np.arange(nB))
    assert np.abs(a - b).max() < 1e-12 and np.abs(la - lb).max() < 1e-12


def test_linearity_in_values():
    H, nB, d = 1, 4, 16
    q = _rand((1, H, nB * 64, d), 80, 2.0)
    k = _rand((1, H, nB * 64, d), 81, 2.0)
    v1 = _rand((1, H, nB * 64, d), 82)
    v2 = _rand((1, H, nB * 64, d), 83)
    rp, ci = _full_csr(nB, nB)
    rows = np.arange(nB)
    o1, _ = oracle.attention_rows(q, k, v1, rp, ci, rows)
    o2, _ = oracle.attention_rows(q, k, v2, rp, ci, rows)
    o3, _ = oracle.attention_rows(q, k, (2 * v1 - 3 * v2).astype(np.float32), rp, ci, rows)
    assert np.abs(o3 - (2 * o1 - 3 * o2)).max() < 1e-5   # fp32 rounding of 2 v1 - 3 v2


def test_single_block_grid_is_dense():
    d = 32
    q = _rand((1, 1, 64, d), 90, 2.0)
    k = _rand((1, 1, 64, d), 91, 2.0)
    v = _rand((1, 1, 64, d), 92)
    mask, rp, ci = oracle.select(q, k, 1, (1, 1, 1), 0.01)
    assert mask.all()
    out, _ = oracle.attention_rows(q, k, v, rp, ci, [0])
    ref, _ = brute.dense_attention(q[0, 0], k[0, 0], v[0, 0], 1 / math.sqrt(d))
    assert np.abs(out[0] - ref).max() < 1e-12


def test_batch_and_head_indexing():
    # two batches x two heads with different data: each (b, h) must use its own slice
    B, H, nB, d = 2, 2, 3, 16
    q = _rand((B, H, nB * 64, d), 95, 2.0)
    k = _rand((B, H, nB * 64, d), 96, 2.0)
    v = _rand((B, H, nB * 64, d), 97)
    thr = [0.5, 0.95]
    mask, rp, ci = oracle.select(q, k, H, (1, 1, nB), thr)
    out, _ = oracle.attention_rows(q, k, v, rp, ci, np.arange(B * H * nB))
    for b in range(B):
        for h in range(H):
            bh = b * H + h
            m1, rp1, ci1 = oracle.select(q[b:b + 1, h:h + 1], k[b:b + 1, h:h + 1], 1, (1, 1, nB), thr[h])
            assert np.array_equal(mask[bh * nB:(bh + 1) * nB], m1)
            o1, _ = oracle.attention_rows(q[b:b + 1, h:h + 1], k[b:b + 1, h:h + 1], v[b:b + 1, h:h + 1],
                                          rp1, ci1, np.arange(nB))
            assert np.array_equal(out[bh * nB:(bh + 1) * nB], o1)


# ---------------------------------------------------------------- token reordering

@pytest.mark.parametrize("grid,tile", [((2, 16, 24), (1, 8, 8)), ((4, 8, 8), (2, 4, 8)), ((3, 8, 16), (1, 8, 8))])
def test_tile_order_groups_each_tile_row_major(grid, tile):
    """Block b holds exactly the tokens of tile b, in row-major order inside the tile."""
    T, H, W = grid
    tt, th, tw = tile
    perm = oracle.tile_order(grid, tile)
    assert np.array_equal(np.sort(perm), np.arange(T * H * W))          # a permutation
    t, y, x = perm // (H * W), (perm // W) % H, perm % W
    vol = tt * th * tw
    nTy, nTx = H // th, W // tw
    for b in range(T * H * W // vol):
        sl = slice(vol * b, vol * (b + 1))
        assert np.all(t[sl] // tt == b // (nTy * nTx))
        assert np.all(y[sl] // th == (b // nTx) % nTy)
        assert np.all(x[sl] // tw == b % nTx)
        key = (t[sl] % tt) * (th * tw) + (y[sl] % th) * tw + x[sl] % tw
        assert np.array_equal(key, np.arange(vol))


def test_tile_order_round_trip_and_input_generator():
    """from_tiles inverts to_tiles, and to_tiles agrees with the input generator's own
    tile-major permutation (written separately, with reshapes)."""
    import torch
    from block_sparse_attention_row_amd.synth import tile_major
    grid, tile = (3, 16, 24), (1, 8, 8)
    rng = np.random.default_rng(4)
    field = rng.standard_normal((2, 3, 5) + grid).astype(np.float32)       # [B, H, d, T, Hh, W]
    x = np.ascontiguousarray(field.reshape(2, 3, 5, -1).transpose(0, 1, 3, 2))   # raster tokens [B, H, N, d]
    y = oracle.to_tiles(x, grid, tile)
    assert np.array_equal(oracle.from_tiles(y, grid, tile), x)
    assert np.array_equal(y, tile_major(torch.from_numpy(field), grid, tile).numpy())


# ---------------------------------------------------------------- gradients

def _loss(q, k, v, g, mask, scale, tpb):
    """sum(g * O) with O from the token-masked brute force (fp64), per head."""
    tot = 0.0
    for h in range(q.shape[0]):
        o, _ = brute.token_mask_attention(q[h], k[h], v[h], mask[h], scale, tpb)
        tot += float(np.sum(g[h] * o))
    return tot


def test_backward_matches_finite_differences():
    """Every gradient entry of a tiny case against central differences of
    sum(dO * O), O from the token-masked brute force (a separate route)."""
    rng = np.random.default_rng(8)
    H, nB, tpb, d = 2, 3, 4, 5
    N = nB * tpb
    q, k, v, g = (rng.standard_normal((H, N, d)).astype(np.float32) for _ in range(4))
    mask = rng.random((H, nB, nB)) < 0.6
    mask[:, np.arange(nB), np.arange(nB)] = True
    mask[1, 2] = False                                  # an empty row
    scale = 0.7
    rp, ci = oracle.csr_from_mask(mask.reshape(H * nB, nB))
    dq, dk, dv = oracle.attention_backward(q[None], k[None], v[None], g[None], rp, ci, scale=scale, tpb=tpb)
    q64, k64, v64, g64 = (x.astype(np.float64) for x in (q, k, v, g))
    h = 1e-6
    for name, x, grad in (("q", q64, dq[0]), ("k", k64, dk[0]), ("v", v64, dv[0])):
        num = np.empty_like(x)
        for idx in np.ndindex(*x.shape):
            xp = x.copy(); xp[idx] += h
            xm = x.copy(); xm[idx] -= h
            args = {"q": q64, "k": k64, "v": v64}
            args[name] = xp
            lp = _loss(args["q"], args["k"], args["v"], g64, mask, scale, tpb)
            args[name] = xm
            lm = _loss(args["q"], args["k"], args["v"], g64, mask, scale, tpb)
            num[idx] = (lp - lm) / (2 * h)
        assert np.abs(num - grad).max() <= 1e-6 * max(1.0, np.abs(num).max()), name


def test_backward_zero_outside_the_kept_blocks():
    """Key blocks kept by no query block get no dK, dV; empty query rows get no dQ."""
    rng = np.random.default_rng(9)
    nB, tpb, d = 4, 8, 6
    N = nB * tpb
    q, k, v, g = (rng.standard_normal((1, 1, N, d)).astype(np.float32) for _ in range(4))
    mask = np.zeros((nB, nB), dtype=bool)
    mask[0, [0, 2]] = True
    mask[2, [2]] = True
    mask[3, [0]] = True                                 # row 1 empty; key block 1 and 3 unused
    rp, ci = oracle.csr_from_mask(mask)
    dq, dk, dv = oracle.attention_backward(q, k, v, g, rp, ci, tpb=tpb)
    for b in (1, 3):
        assert np.all(dk[0, 0, b * tpb:(b + 1) * tpb] == 0) and np.all(dv[0, 0, b * tpb:(b + 1) * tpb] == 0)
    assert np.all(dq[0, 0, tpb:2 * tpb] == 0)
    assert np.abs(dq).max() > 0 and np.abs(dk).max() > 0 and np.abs(dv).max() > 0


def test_backward_with_stored_output():
    """D = dO . O uses the caller's stored output when given.  Shifting O by delta
    shifts D by dO . delta, which leaves dV unchanged and moves dQ_n by
    -scale (dO_n . delta_n) sum_m P_nm k_m (closed form; P k from the brute force
    with k as the values)."""
    rng = np.random.default_rng(10)
    H, nB, tpb, d = 2, 3, 4, 5
    N = nB * tpb
    q, k, v, g = (rng.standard_normal((H, N, d)).astype(np.float32) for _ in range(4))
    mask = rng.random((H, nB, nB)) < 0.6
    mask[:, np.arange(nB), np.arange(nB)] = True
    scale = 0.6
    rp, ci = oracle.csr_from_mask(mask.reshape(H * nB, nB))
    ref = oracle.attention_backward(q[None], k[None], v[None], g[None], rp, ci, scale=scale, tpb=tpb)
    o = np.stack([brute.token_mask_attention(q[h].astype(np.float64), k[h].astype(np.float64),
                                             v[h].astype(np.float64), mask[h], scale, tpb)[0] for h in range(H)])
    same = oracle.attention_backward(q[None], k[None], v[None], g[None], rp, ci, scale=scale, tpb=tpb,
                                     out=o[None].astype(np.float32))
    for a, b in zip(same, ref):
        assert np.abs(a - b).max() <= 1e-6 * np.abs(b).max()
    delta = rng.standard_normal((H, N, d)).astype(np.float32)
    shifted = (o.astype(np.float32) + delta)
    got = oracle.attention_backward(q[None], k[None], v[None], g[None], rp, ci, scale=scale, tpb=tpb,
                                    out=shifted[None])
    assert np.array_equal(got[2], same[2])
    dD = np.sum(g.astype(np.float64) * (shifted.astype(np.float64) - o.astype(np.float32)), axis=-1)   # [H, N]
    pk = np.stack([brute.token_mask_attention(q[h].astype(np.float64), k[h].astype(np.float64),
                                              k[h].astype(np.float64), mask[h], scale, tpb)[0] for h in range(H)])
    expect = same[0][0] - scale * dD[..., None] * pk
    assert np.abs(got[0][0] - expect).max() <= 1e-9 * np.abs(expect).max()


# ---------------------------------------------------------------- sampling with inclusion probabilities (SIP)

def test_splitmix64_reference_values():
    from oracle import sip
    path = os.path.join(os.path.dirname(__file__), "golden", "splitmix64_seed0.txt")
    rows = [ln.split() for ln in open(path) if ln.strip() and not ln.startswith("#")]
    for cnt, hexv in rows:
        assert int(sip.splitmix64(0, int(cnt))) == int(hexv, 16)


def test_uniforms_are_24_bit_and_indexed_by_row_and_block():
    from oracle import sip
    u = sip.uniforms(7, 3, 5)
    assert u.shape == (3, 5) and np.all((u >= 0) & (u < 1))
    assert np.all(u * 2 ** 24 == np.floor(u * 2 ** 24))
    # row r, block j is output r * nB + j + 1 of the stream
    z = int(sip.splitmix64(7, 2 * 5 + 3 + 1))
    assert u[2, 3] == (z >> 40) * 2.0 ** -24
    assert np.array_equal(sip.uniforms(7, 2, 5, row0=1), u[1:])


def test_inclusion_probabilities_closed_forms():
    from oracle import sip
    # uniform scores: pi = k / n everywhere
    assert np.allclose(sip.inclusion_probabilities(np.full(8, 1 / 8), 3.0), 3 / 8, rtol=0, atol=1e-15)
    # two blocks, k = 1.5: a >= 2/3 caps the first block (pi = 1, 0.5); below, pi = 1.5 p
    for a in (0.9, 2 / 3 + 1e-9, 0.6, 0.5):
        pi = sip.inclusion_probabilities(np.array([a, 1 - a]), 1.5)[0]
        want = np.array([1.0, 0.5]) if 1.5 * a >= 1 else 1.5 * np.array([a, 1 - a])
        assert np.allclose(pi, want, rtol=0, atol=1e-12), (a, pi)
    # p = (1/2, 1/4, 1/8, 1/8), k = 2: c = 2 caps block 0; then c = 1 / (1/2) = 2 for the
    # rest -> (1, 1/2, 1/4, 1/4)
    pi = sip.inclusion_probabilities(np.array([0.5, 0.25, 0.125, 0.125]), 2.0)[0]
    assert np.allclose(pi, np.array([1.0, 0.5, 0.25, 0.25]), rtol=0, atol=1e-15)
    # budget at least the positive count keeps every positive block, never a zero one
    pi = sip.inclusion_probabilities(np.array([0.7, 0.3, 0.0]), 2.0)[0]
    assert np.array_equal(pi, np.array([1.0, 1.0, 0.0]))


def test_inclusion_probabilities_invariants():
    from oracle import sip
    rng = np.random.default_rng(21)
    p = rng.gamma(0.3, size=(40, 50))
    p /= p.sum(axis=1, keepdims=True)
    for k in (1.0, 4.5, 12.0, 49.0):
        pi = sip.inclusion_probabilities(p, k)
        assert np.allclose(pi.sum(axis=1), k, rtol=0, atol=1e-9)
        assert np.all(pi <= 1.0) and np.all(pi >= 0.0)
        for r in range(p.shape[0]):
            free = pi[r] < 1.0
            if free.sum() >= 2:                          # uncapped blocks: pi proportional to p
                ratio = pi[r][free] / p[r][free]
                assert np.allclose(ratio, ratio[0], rtol=1e-12)
                assert p[r][~free].min(initial=np.inf) >= p[r][free].max()   # capped = the largest
        perm = rng.permutation(p.shape[1])
        assert np.allclose(sip.inclusion_probabilities(p[:, perm], k), pi[:, perm], rtol=0, atol=1e-12)


def test_sampling_frequency_and_horvitz_thompson():
    """Over many independent rows of the same scores, block j is kept with frequency
    pi_j, and sum over kept blocks of x_j / pi_j averages to sum_j x_j."""
    from oracle import sip
    p = np.array([0.4, 0.2, 0.15, 0.1, 0.08, 0.04, 0.02, 0.01])
    k = 3.0
    pi = sip.inclusion_probabilities(p, k)[0]
    R = 20000
    u = sip.uniforms(5, R, p.size)
    keep = u < pi
    freq = keep.mean(axis=0)
    sd = np.sqrt(pi * (1 - pi) / R)
    assert np.all(np.abs(freq - pi) <= 5 * sd + 1e-12)
    x = np.linspace(1.0, 2.0, p.size)
    ht = (keep * (x / pi)).sum(axis=1)
    assert abs(ht.mean() - x.sum()) <= 5 * ht.std() / np.sqrt(R)


def test_logit_offset_zero_or_constant_changes_nothing():
    rng = np.random.default_rng(30)
    nB, tpb, d = 3, 8, 4
    N = nB * tpb
    q, k, v = (rng.standard_normal((1, 1, N, d)).astype(np.float32) for _ in range(3))
    mask = rng.random((nB, nB)) < 0.7
    mask[np.arange(nB), np.arange(nB)] = True
    rp, ci = oracle.csr_from_mask(mask)
    rows = np.arange(nB)
    o0, l0 = oracle.attention_rows(q, k, v, rp, ci, rows, tpb=tpb)
    o1, l1 = oracle.attention_rows(q, k, v, rp, ci, rows, tpb=tpb, bias=np.zeros(len(ci)))
    assert np.array_equal(o0, o1) and np.array_equal(l0, l1)
    # one constant per row: the softmax is unchanged, the LSE moves by it
    cst = np.repeat(np.array([0.3, -1.2, 2.0]), np.diff(rp))
    o2, l2 = oracle.attention_rows(q, k, v, rp, ci, rows, tpb=tpb, bias=cst)
    assert np.allclose(o2, o0, rtol=0, atol=1e-12)
    assert np.allclose(l2 - l0, np.array([0.3, -1.2, 2.0])[:, None], rtol=0, atol=1e-12)


def test_logit_offset_ln_w_equals_w_copies_of_the_block():
    """An offset ln(w) on a block (w integer) is the block's keys listed w times:
    checked against token-level brute force on a key set with the copies appended."""
    rng = np.random.default_rng(31)
    nB, tpb, d = 3, 4, 5
    N = nB * tpb
    q, k, v = (rng.standard_normal((N, d)) for _ in range(3))
    mask = np.array([[1, 1, 0], [0, 1, 1], [1, 1, 1]], dtype=bool)
    w = {(0, 1): 3, (1, 2): 2, (2, 0): 4}                 # (row, block) -> copies
    rp, ci = oracle.csr_from_mask(mask)
    bias = np.zeros(len(ci))
    for r in range(nB):
        for e in range(rp[r], rp[r + 1]):
            bias[e] = math.log(w.get((r, int(ci[e])), 1))
    out, _ = oracle.attention_rows(q[None, None].astype(np.float32), k[None, None].astype(np.float32),
                                   v[None, None].astype(np.float32), rp, ci, np.arange(nB), tpb=tpb, scale=0.5,
                                   bias=bias)
    q32, k32, v32 = (x.astype(np.float32).astype(np.float64) for x in (q, k, v))
    for r in range(nB):
        keys, vals = [], []
        for j in range(nB):
            if mask[r, j]:
                for _ in range(w.get((r, j), 1)):
                    keys.append(k32[j * tpb:(j + 1) * tpb])
                    vals.append(v32[j * tpb:(j + 1) * tpb])
        K, V = np.concatenate(keys), np.concatenate(vals)
        ref, _ = brute.dense_attention(q32[r * tpb:(r + 1) * tpb], K, V, 0.5)
        assert np.allclose(out[r], ref, rtol=0, atol=1e-12)


def test_select_sip_consistency():
    """The sampled list is u < pi with offsets -ln(pi) of the kept blocks, and a budget
    of all blocks keeps everything with zero offsets."""
    from oracle import sip
    rng = np.random.default_rng(32)
    q = rng.standard_normal((1, 2, 6 * 64, 8)).astype(np.float32)
    k = (q + 0.3 * rng.standard_normal(q.shape)).astype(np.float32)
    keep, rp, ci, bias, pi, u = sip.select_sip(q, k, 2, 2.5, seed=9)
    assert np.array_equal(keep, u < pi)
    assert np.allclose(pi.sum(axis=1), 2.5, rtol=0, atol=1e-9)
    r = np.repeat(np.arange(keep.shape[0]), np.diff(rp))
    assert np.array_equal(bias, -np.log(pi[r, ci]))
    keep, rp, ci, bias, pi, u = sip.select_sip(q, k, 2, 6.0, seed=9)
    assert keep.all() and np.all(bias == 0)


def test_inclusion_probabilities_from_scores_shift_and_range():
    """pi depends on the scores only through their differences, and blocks far below the
    row maximum still receive the budget the capped ones leave (no underflow): one
    dominant block plus three equal ones 2000 nats lower, budget 2 -> (1, 1/3, 1/3, 1/3)."""
    from oracle import sip
    s = np.array([[0.0, -2000.0, -2000.0, -2000.0]])
    pi = sip.inclusion_probabilities_from_scores(s, 2.0)
    assert np.allclose(pi, [[1.0, 1 / 3, 1 / 3, 1 / 3]], rtol=0, atol=1e-15)
    rng = np.random.default_rng(33)
    s = rng.normal(scale=5.0, size=(6, 30))
    a = sip.inclusion_probabilities_from_scores(s, 7.0)
    b = sip.inclusion_probabilities_from_scores(s + 123.0, 7.0)
    assert np.allclose(a, b, rtol=0, atol=1e-12)
    assert np.allclose(a, sip.inclusion_probabilities(np.exp(s - s.max(1, keepdims=True)) /
                                                      np.exp(s - s.max(1, keepdims=True)).sum(1, keepdims=True), 7.0),
                       rtol=0, atol=1e-12)


# ---------------------------------------------------------------- DynamicRad radial window

def test_radial_radii_by_hand():
    from oracle import radial
    # r0 = 4, gamma = 1/2: widths 4, 2, 1, 0.5, 0.25, ... -> radii 4, 2, 1, then skipped
    assert radial.radii(6, 4.0, 0.5, 0).tolist() == [4, 2, 1, -1, -1, -1]
    # lambda = 2: skipped frames at even distance keep the co-located block
    assert radial.radii(7, 4.0, 0.5, 2).tolist() == [4, 2, 1, -1, 0, -1, 0]
    # r0 below 1: the own frame still keeps its block
    assert radial.radii(3, 0.5, 0.9, 0).tolist() == [0, -1, -1]
    # gamma = 1: a constant radius
    assert radial.radii(4, 2.7, 1.0, 0).tolist() == [2, 2, 2, 2]


def test_radial_with_gamma_one_is_a_box_window():
    """gamma = 1, lambda = 0: the clipped box over all frames and +-floor(r0) tiles,
    counted by the brute-force window counter."""
    from oracle import radial
    grid = (3, 5, 6)
    m = radial.radial_mask(grid, 1.5, 1.0, 0)
    for i in range(m.shape[0]):
        assert m[i].sum() == brute.window_count(i, grid, (grid[0], 1, 1))


def test_radial_counts_closed_form_and_symmetry():
    """An interior block of a large grid keeps (2R(0)+1)^2 + 2 sum_{dt>0} (2R(dt)+1)^2
    blocks over the frames with R >= 0; the mask is symmetric."""
    from oracle import radial
    grid = (9, 13, 13)
    r0, g, lam = 5.0, 0.6, 3
    m = radial.radial_mask(grid, r0, g, lam)
    R = radial.radii(grid[0], r0, g, lam)
    centre = 4 * 13 * 13 + 6 * 13 + 6
    want = (2 * R[0] + 1) ** 2 + 2 * sum((2 * R[dt] + 1) ** 2 for dt in range(1, 5) if R[dt] >= 0)
    assert m[centre].sum() == want
    assert np.array_equal(m, m.T)


# ---------------------------------------------------------------- intra-block clustering selector (IBCS)

def test_kmeans_recovers_separated_clusters():
    """Eight tight, well separated groups (sizes 4 .. 32) laid out so that the start
    positions n*c/8 fall in distinct groups: centroids are the group means and the
    weights their shares after the first round."""
    from oracle import ibcs
    rng = np.random.default_rng(40)
    sizes = [16] * 8
    centres = rng.normal(scale=50.0, size=(8, 6))
    x = np.concatenate([centres[c] + 0.01 * rng.normal(size=(sizes[c], 6)) for c in range(8)])
    mu, w, gap = ibcs.kmeans(x)
    starts = np.cumsum([0] + sizes[:-1])
    for c in range(8):
        assert np.allclose(mu[c], x[starts[c]:starts[c] + sizes[c]].mean(axis=0), rtol=0, atol=1e-12)
    assert np.allclose(w, np.array(sizes) / sum(sizes))
    assert gap > 0.9


def test_kmeans_identical_points_and_ties():
    """All queries equal: every distance ties, everything goes to cluster 0 (lower
    index), the empty clusters keep their (equal) starting centroids."""
    from oracle import ibcs
    x = np.tile(np.array([1.0, -2.0, 0.5]), (128, 1))
    mu, w, gap = ibcs.kmeans(x)
    assert np.array_equal(w, np.eye(8)[0]) and np.allclose(mu, x[0]) and gap == 0.0


def test_ibcs_reduces_to_nabla_when_a_block_is_constant():
    """Identical queries inside each 128-token block: one cluster of weight 1 whose
    centroid is the block mean, so p~ is the softmax of the pooled scores (formed
    here from the raw tokens, by brute force)."""
    from oracle import ibcs
    rng = np.random.default_rng(41)
    nB, d = 5, 8
    base = rng.normal(size=(3, d))
    q = np.repeat(base, 128, axis=0)[: nB * 64][None, None].astype(np.float32)
    k = rng.normal(size=(1, 1, nB * 64, d)).astype(np.float32)
    pt, gaps = ibcs.mixture_scores(q, k, 1)
    kbar = k[0, 0].astype(np.float64).reshape(nB, 64, d).mean(axis=1)
    for i in range(nB):
        s = base[i // 2].astype(np.float32).astype(np.float64) @ kbar.T / math.sqrt(d)
        ref = np.exp(s - s.max()) / np.exp(s - s.max()).sum()
        assert np.allclose(pt[i], ref, rtol=0, atol=1e-14)


def test_ibcs_rows_are_distributions_shared_by_the_pair():
    from oracle import ibcs
    rng = np.random.default_rng(42)
    q = rng.normal(size=(1, 2, 5 * 64, 16)).astype(np.float32)
    k = rng.normal(size=(1, 2, 5 * 64, 16)).astype(np.float32)
    pt, gaps = ibcs.mixture_scores(q, k, 2)
    assert np.allclose(pt.sum(axis=1), 1.0, rtol=0, atol=1e-12)
    for h in range(2):
        for p in range(2):
            assert np.array_equal(pt[h * 5 + 2 * p], pt[h * 5 + 2 * p + 1])
    assert gaps.shape == (2, 3)


def test_cdf_keep_against_pairwise_brute_force():
    from oracle import ibcs
    rng = np.random.default_rng(43)
    p = rng.gamma(0.5, size=(30, 17))
    p[:, 3] = p[:, 5]                               # exact ties
    p /= p.sum(axis=1, keepdims=True)
    for thr in (0.3, 0.8, 0.95):
        keep = ibcs.cdf_keep(p, thr)
        for r in range(p.shape[0]):
            assert np.array_equal(keep[r], brute.cdf_keep_pairwise(p[r], thr).astype(bool))
    assert ibcs.cdf_keep(p, 1.0).all()


def _kmeans_chain_golden():
    chain, rounds = None, {}
    with open(os.path.join(os.path.dirname(__file__), "golden", "kmeans_chain.txt")) as f:
        for line in f:
            tok = line.split()
            if not tok or tok[0].startswith("#"):
                continue
            if tok[0] == "chain":
                chain = [float(v) for v in tok[1:]]
            elif tok[0] == "rounds":
                r, a, b, c, d, n0, n1 = (int(v) for v in tok[1:])
                rounds[r] = (a / b, c / d, n0, n1)
    x = np.zeros((128, 3))
    x[:32, 0] = chain
    for g in range(2, 8):
        x[16 * g:16 * g + 16, 0] = 1024.0 * g
    return x, rounds


def test_kmeans_round_count_against_hand_derived_chain():
    """The k-means runs exactly ITERS = 4 rounds: on a chain that moves in every one of
    its first nine rounds, the oracle's centroids and weights equal the hand-derived
    values after round 4 (tests/golden/kmeans_chain.txt), and running 1, 2, 3 or 5
    rounds gives the hand-derived values of those rounds, which all differ from
    round 4's.  The tie of the first round (three points at the midpoint) goes to
    the lower cluster."""
    from oracle import ibcs
    x, rounds = _kmeans_chain_golden()
    assert ibcs.ITERS == 4
    for r, (m0, m1, n0, n1) in rounds.items():
        mu, w, gap = ibcs.kmeans(x, iters=r)
        assert abs(mu[0, 0] - m0) <= 1e-12 and abs(mu[1, 0] - m1) <= 1e-12, r
        assert np.all(mu[:, 1:] == 0.0)
        assert np.array_equal(mu[2:, 0], 1024.0 * np.arange(2, 8))
        assert w[0] * 128 == n0 and w[1] * 128 == n1 and np.all(w[2:] * 128 == 16)
        if r != 4:
            assert (m0, m1) != rounds[4][:2]
    mu, w, gap = ibcs.kmeans(x)
    m0, m1, n0, n1 = rounds[4]
    assert abs(mu[0, 0] - m0) <= 1e-12 and abs(mu[1, 0] - m1) <= 1e-12
    assert w[0] * 128 == n0 and w[1] * 128 == n1
    assert gap == 0.0                                  # the first round's tie



# ---------------------------------------------------------------- partial tiles
# Grids that are not a whole number of tiles (NABLA summary page, "Fractal Flattening":
# patches are grouped whatever the global size of the video): the last tile along y or
# x holds fewer tokens, and its remaining slots in the tile-major layout are padding.

PARTIAL = [((2, 12, 20), (1, 8, 8)), ((3, 9, 17), (1, 8, 8)), ((5, 8, 8), (4, 4, 4)), ((2, 13, 11), (1, 8, 8))]


@pytest.mark.parametrize("grid,tile", PARTIAL)
def test_partial_tile_order_counts(grid, tile):
    """Every raster token appears exactly once; a tile holds prod(min(tile, rest of the
    grid)) tokens along each axis (closed form), the rest of its slots are padding."""
    perm = oracle.tile_order(grid, tile)
    nT, nTy, nTx = oracle.block_grid(grid, tile)
    assert len(perm) == nT * nTy * nTx * 64
    assert np.array_equal(np.sort(perm[perm >= 0]), np.arange(np.prod(grid)))
    valid = oracle.token_valid(grid, tile).reshape(-1, 64)
    for b in range(nT * nTy * nTx):
        bt, by, bx = b // (nTy * nTx), (b // nTx) % nTy, b % nTx
        n = (min(tile[0], grid[0] - bt * tile[0]) * min(tile[1], grid[1] - by * tile[1])
             * min(tile[2], grid[2] - bx * tile[2]))
        assert valid[b].sum() == n


@pytest.mark.parametrize("grid,tile", PARTIAL)
def test_partial_tiles_round_trip_and_pool(grid, tile):
    """to_tiles / from_tiles invert each other and pad with zeros; the pooled mean of a
    partial tile is the mean of the grid tokens inside it, taken here by slicing the
    raster grid directly (no tile-major order involved)."""
    T, H, W = grid
    x = _rand((2, T * H * W, 8), 61)
    xt = oracle.to_tiles(x, grid, tile)
    valid = oracle.token_valid(grid, tile)
    assert np.all(xt[:, ~valid] == 0)
    assert np.array_equal(oracle.from_tiles(xt, grid, tile), x)
    pooled = oracle.pool(xt, valid=valid)
    nT, nTy, nTx = oracle.block_grid(grid, tile)
    xr = x.astype(np.float64).reshape(2, T, H, W, 8)
    for b in range(nT * nTy * nTx):
        bt, by, bx = b // (nTy * nTx), (b // nTx) % nTy, b % nTx
        sl = xr[:, bt * tile[0]:(bt + 1) * tile[0], by * tile[1]:(by + 1) * tile[1], bx * tile[2]:(bx + 1) * tile[2]]
        assert np.allclose(pooled[:, b], sl.reshape(2, -1, 8).mean(axis=1), rtol=0, atol=1e-12)


@pytest.mark.parametrize("grid,tile", PARTIAL[:3])
def test_partial_tile_walk_matches_raster_bruteforce(grid, tile):
    """The tile walk over the padded tile-major layout, with padding keys left out and
    padding queries zero, equals masked dense attention on the raster grid whose mask
    comes from each token's own block coordinates."""
    T, H, W = grid
    n, d = T * H * W, 16
    q, k, v = (_rand((1, 1, n, d), s) for s in (62, 63, 64))
    qt, kt, vt = (oracle.to_tiles(a, grid, tile) for a in (q, k, v))
    # padding slots hold junk: it must not matter
    valid = oracle.token_valid(grid, tile)
    for a in (qt, kt, vt):
        a[..., ~valid, :] = 7.0
    nB = int(np.prod(oracle.block_grid(grid, tile)))
    mask = np.random.default_rng(65).random((nB, nB)) < 0.6
    mask[np.arange(nB), np.arange(nB)] = True
    rp, ci = oracle.csr_from_mask(mask)
    sc = 1.0 / math.sqrt(d)
    out, lse = oracle.attention_rows(qt, kt, vt, rp, ci, np.arange(nB), scale=sc, valid=valid)
    ref, ref_lse = brute.raster_block_mask_attention(q[0, 0], k[0, 0], v[0, 0], grid, tile, mask, sc)
    perm = oracle.tile_order(grid, tile)
    got = out.reshape(-1, d)
    got_l = lse.reshape(-1)
    assert np.allclose(got[valid], ref[perm[valid]], rtol=0, atol=1e-12)
    assert np.allclose(got_l[valid], ref_lse[perm[valid]], rtol=0, atol=1e-12)
    assert np.all(got[~valid] == 0) and np.all(np.isneginf(got_l[~valid]))


def test_backward_partial_tiles_match_raster_finite_differences():
    """Partial tiles in the backward: on the padded tile-major layout (junk in every
    padding slot, dO included) the gradients are zero at padding slots, and at token
    slots equal central differences of sum(dO * O) with O the masked dense attention
    on the raster grid (blocks from each token's grid coordinates, no tile-major order)."""
    grid, tile = (1, 9, 10), (1, 8, 8)
    n, d = 90, 4
    q, k, v, g = (_rand((n, d), s).astype(np.float64) for s in (81, 82, 83, 84))
    nB = int(np.prod(oracle.block_grid(grid, tile)))
    mask = np.random.default_rng(85).random((nB, nB)) < 0.6
    mask[np.arange(nB), np.arange(nB)] = True
    mask[1, 3] = mask[3, 1] = True
    rp, ci = oracle.csr_from_mask(mask)
    sc = 0.45
    valid = oracle.token_valid(grid, tile)
    tiled = [oracle.to_tiles(a.astype(np.float32)[None, None], grid, tile) for a in (q, k, v, g)]
    for a in tiled:
        a[..., ~valid, :] = 7.0
    dq, dk, dv = oracle.attention_backward(*tiled, rp, ci, scale=sc, valid=valid)
    for gr in (dq, dk, dv):
        assert np.all(gr[0, 0, ~valid] == 0)
    perm = oracle.tile_order(grid, tile)

    def loss(qq, kk, vv):
        o, _ = brute.raster_block_mask_attention(qq, kk, vv, grid, tile, mask, sc)
        return float(np.sum(g.astype(np.float32).astype(np.float64) * o))

    q32, k32, v32 = (a.astype(np.float32).astype(np.float64) for a in (q, k, v))
    h = 1e-6
    for name, grad in (("q", dq), ("k", dk), ("v", dv)):
        num = np.empty((n, d))
        for i in range(n):
            for c in range(d):
                args = {"q": q32.copy(), "k": k32.copy(), "v": v32.copy()}
                args[name][i, c] += h
                lp = loss(args["q"], args["k"], args["v"])
                args[name][i, c] -= 2 * h
                lm = loss(args["q"], args["k"], args["v"])
                num[i, c] = (lp - lm) / (2 * h)
        got = np.empty((n, d))
        got[perm[valid]] = grad[0, 0][valid]
        assert np.abs(got - num).max() <= 1e-6 * max(1.0, np.abs(num).max()), name


def test_whole_tiles_need_no_padding():
    """A grid of whole tiles has no padding slot and the same order as before."""
    grid, tile = (2, 16, 24), (1, 8, 8)
    perm = oracle.tile_order(grid, tile)
    assert (perm >= 0).all() and len(perm) == 2 * 16 * 24
    x = _rand((1, len(perm), 4), 66)
    assert np.array_equal(oracle.pool(x), oracle.pool(x, valid=oracle.token_valid(grid, tile)))



# ---------------------------------------------------------------- 4-token key blocks (AB-Attention)
# AB-Attention page, "Les trois techniques d'AB-Attention", third technique: key and
# value blocks of 4 tokens, the kept ones gathered by index into full tiles.

def test_four_token_blocks_of_a_whole_tile_equal_the_tile():
    """Listing all 16 four-token blocks of a 64-token tile gives the same attention as
    listing the tile itself."""
    rng = np.random.default_rng(81)
    nB, d = 6, 32
    q, k, v = (_rand((1, 2, nB * 64, d), s) for s in (82, 83, 84))
    mask = rng.random((2 * nB, nB)) < 0.5
    mask[:, 0] = True
    rp, ci = oracle.csr_from_mask(mask)
    fine = np.repeat(mask, 16, axis=1)                      # block j -> sub-blocks 16 j .. 16 j + 15
    rp4, ci4 = oracle.csr_from_mask(fine)
    rows = np.arange(2 * nB)
    o, l = oracle.attention_rows(q, k, v, rp, ci, rows)
    o4, l4 = oracle.attention_rows(q, k, v, rp4, ci4, rows, key_tokens=4)
    assert np.allclose(o4, o, rtol=0, atol=1e-12) and np.allclose(l4, l, rtol=0, atol=1e-12)


def test_four_token_gather_matches_token_mask_bruteforce():
    rng = np.random.default_rng(85)
    nB, d = 5, 16
    q, k, v = (_rand((1, 1, nB * 64, d), s) for s in (86, 87, 88))
    mask = rng.random((nB, nB * 16)) < 0.3
    mask[2] = False                                          # an empty row
    rp, ci = oracle.csr_from_mask(mask)
    sc = 1.0 / math.sqrt(d)
    out, lse = oracle.attention_rows(q, k, v, rp, ci, np.arange(nB), scale=sc, key_tokens=4)
    ref, ref_lse = brute.token_mask_attention(q[0, 0], k[0, 0], v[0, 0], mask, sc, tpb=64, key_tokens=4)
    assert np.allclose(out.reshape(-1, d), ref, rtol=0, atol=1e-12)
    assert np.array_equal(np.isneginf(lse.reshape(-1)), np.isneginf(ref_lse))
    fin = np.isfinite(ref_lse)
    assert np.allclose(lse.reshape(-1)[fin], ref_lse[fin], rtol=0, atol=1e-12)


def test_fine_selection_against_pairwise_cdf():
    """The rows of the 4-token selection are the CDF rule (pairwise brute force) on the
    softmax of 64-token query means against 4-token key means, both taken here by
    reshape-means; thr >= 1 keeps every key block."""
    nB, d, H = 4, 16, 2
    q = _rand((1, H, nB * 64, d), 89, 0.5)
    k = _rand((1, H, nB * 64, d), 90, 0.5)
    thr = np.array([0.6, 0.85])
    keep, rp, ci = oracle.select_fine(q, k, H, thr)
    assert keep.shape == (H * nB, nB * 16)
    qb = q.astype(np.float64).reshape(H, nB, 64, d).mean(axis=2)
    kb = k.astype(np.float64).reshape(H, nB * 16, 4, d).mean(axis=2)
    for h in range(H):
        s = qb[h] @ kb[h].T / math.sqrt(d)
        p = np.exp(s - s.max(axis=1, keepdims=True))
        p /= p.sum(axis=1, keepdims=True)
        for i in range(nB):
            assert np.array_equal(keep[h * nB + i], brute.cdf_keep_pairwise(p[i], thr[h]).astype(bool))
    assert oracle.select_fine(q, k, H, 1.0)[0].all()
