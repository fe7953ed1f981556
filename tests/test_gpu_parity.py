"""GPU parity: the HIP path (through the C-ABI) against the CPU oracle.

Small workloads (several tiles, ragged block counts, both dtypes and head
sizes, windows, per-head thresholds, batch > 1) are compared in full; the
five full-size workloads in test_gpu_workloads.py.
"""
import numpy as np
import pytest
import torch

import oracle
from block_sparse_attention_row_amd import binding as B
from block_sparse_attention_row_amd.synth import WORKLOADS, make_inputs, small_workload

from . import parity as P

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a ROCm GPU")
    B.lib()


SMALL = [
    # name, heads, d, block grid, dtype, thr, window, reading, head-thr range, batch
    ("f32_d64_tiny", 1, 64, (4, 2, 2), "f32", 0.9, (-1, -1, -1), "A", None, 1),
    ("f32_d128_ragged", 2, 128, (3, 3, 5), "f32", 0.8, (-1, -1, -1), "B", None, 1),
    ("bf16_d128_ragged", 3, 128, (3, 5, 7), "bf16", 0.85, (-1, -1, -1), "A", None, 1),
    ("bf16_d128_sparse", 2, 128, (4, 4, 6), "bf16", 0.9, (-1, -1, -1), "B", None, 1),
    ("bf16_d64_window", 2, 64, (2, 3, 5), "bf16", 0.7, (1, 1, 1), "B", None, 1),
    ("bf16_d128_window_A", 2, 128, (5, 3, 4), "bf16", 0.8, (1, 1, 1), "A", None, 1),
    ("bf16_d128_headthr", 4, 128, (2, 4, 9), "bf16", 0.7, (-1, -1, -1), "A", (0.6, 0.8), 2),
    ("bf16_d128_page", 3, 128, (4, 6, 8), "bf16", 0.9, (-1, -1, -1), "page", None, 1),
    ("bf16_d128_dense", 2, 128, (2, 3, 3), "bf16", 1.0, (-1, -1, -1), "A", None, 1),
    ("bf16_d128_one_block", 2, 128, (1, 1, 1), "bf16", 0.5, (-1, -1, -1), "A", None, 1),
    # one frame of 35 blocks: the forward pairs blocks side by side, the last alone
    ("bf16_d128_one_frame", 2, 128, (1, 5, 7), "bf16", 0.85, (-1, -1, -1), "A", None, 1),
]


def _wl(case):
    name, H, d, bg, dt, thr, win, reading, hr, batch = case
    wl = small_workload(name, H, d, bg, dt, threshold=thr, window=win, head_threshold_range=hr, seed=7)
    return wl.with_(batch=batch), reading


@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
def test_small_select_and_forward(case):
    wl, reading = _wl(case)
    print(f"\n[case] {wl.name} reading={reading} heads={wl.heads} d={wl.head_dim} blocks={wl.blocks}", flush=True)
    q, k, v, thr = make_inputs(wl, reading)
    qd, kd, vd = P.to_device(q, k, v)

    # selection: GPU mask vs oracle mask under the excuse rules
    rp, ci = P.gpu_select(wl, qd, kd, thr)
    gmask = P.check_csr(rp, ci, wl.blocks)
    qbar, kbar, keep, band = P.oracle_select_full(wl, q, k, thr, count_band=True)
    rep = P.compare_masks(gmask, keep, qbar, kbar, wl, thr, band=band)
    P.record_masks(f"small_{wl.name}_{reading}", rep)
    assert P.mask_ok(rep), P.fmt(rep)

    # forward under the oracle's CSR, every row
    orp, oci = oracle.csr_from_mask(keep != 0)
    out, lse = P.gpu_forward(wl, qd, kd, vd, orp, oci)
    rows = np.arange(wl.batch * wl.heads * wl.blocks)
    err, lerr = P.compare_rows(wl, out, lse, q, k, v, orp, oci, rows)
    print(f"forward max|err|={err:.3e} lse max|err|={lerr:.3e}", flush=True)
    tol, ltol = P.forward_tols(wl.dtype, reading)
    assert err <= tol and lerr <= ltol

    # end to end: GPU CSR into GPU forward, on rows where the masks agree
    out2, lse2 = P.gpu_forward(wl, qd, kd, vd, rp, ci)
    same = np.nonzero(~(gmask != (keep != 0)).any(axis=1))[0]
    err2, lerr2 = P.compare_rows(wl, out2, lse2, q, k, v, orp, oci, same)
    assert err2 <= tol and lerr2 <= ltol


LONG_ROWS = [
    # name, heads, d, block grid, thr, window, reading, head-thr range: rows of more than 512
    # blocks (the cut's bracket is compacted), block counts that are not whole 16-key groups
    ("d128_756", 2, 128, (3, 12, 21), 0.8, (-1, -1, -1), "A", None),
    ("d64_720_window", 2, 64, (2, 18, 20), 0.7, (1, 1, 1), "B", None),
    ("d128_1080_window_headthr", 3, 128, (4, 15, 18), 0.9, (1, 2, 2), "A", (0.6, 0.95)),
]


@pytest.mark.parametrize("case", LONG_ROWS, ids=[c[0] for c in LONG_ROWS])
def test_long_row_selection_matches_oracle(case):
    """Selection on rows longer than 512 blocks, every row against the oracle."""
    name, H, d, bg, thr, win, reading, hr = case
    wl = small_workload(name, H, d, bg, "bf16", threshold=thr, window=win, head_threshold_range=hr, seed=19)
    print(f"\n[case] long rows {name} blocks={wl.blocks}", flush=True)
    q, k, _, thr_h = make_inputs(wl, reading)
    qd, kd = P.to_device(q, k)
    rp, ci = P.gpu_select(wl, qd, kd, thr_h)
    gmask = P.check_csr(rp, ci, wl.blocks)
    qbar, kbar, keep, band = P.oracle_select_full(wl, q, k, thr_h, count_band=True)
    rep = P.compare_masks(gmask, keep, qbar, kbar, wl, thr_h, band=band)
    P.record_masks(f"long_rows_{name}", rep)
    assert P.mask_ok(rep), P.fmt(rep)


def test_threshold_one_is_dense_attention():
    wl = small_workload("dense", 2, 128, (2, 2, 3), "bf16", threshold=1.0, seed=3)
    q, k, v, thr = make_inputs(wl, "B")
    qd, kd, vd = P.to_device(q, k, v)
    rp, ci = P.gpu_select(wl, qd, kd, thr)
    gmask = P.check_csr(rp, ci, wl.blocks)
    assert gmask.all()
    out, lse = P.gpu_forward(wl, qd, kd, vd, rp, ci)
    ref = torch.nn.functional.scaled_dot_product_attention(q.double(), k.double(), v.double())
    assert (out.double().cpu() - ref).abs().max().item() <= P.TOL["bf16"]


def test_external_mask_empty_rows_and_roundtrip():
    wl = small_workload("ext", 2, 128, (2, 3, 4), "bf16", seed=11)
    q, k, v, _ = make_inputs(wl, "A")
    qd, kd, vd = P.to_device(q, k, v)
    rng = np.random.default_rng(5)
    rows, nB = wl.heads * wl.blocks, wl.blocks
    mask = rng.random((rows, nB)) < 0.3
    mask[[0, 7, rows - 1]] = False                  # empty rows
    mask[3] = True                                  # a full row
    shape = P.shape_for(wl)
    mdev = torch.as_tensor(mask.astype(np.uint8)).cuda()
    rp, ci = B.sparse_attn_mask_to_csr(shape, mdev)
    torch.cuda.synchronize()
    rp_h = rp.cpu().numpy().astype(np.int64)
    ci_h = ci[:int(rp_h[-1])].cpu().numpy()
    orp, oci = oracle.csr_from_mask(mask)
    assert np.array_equal(rp_h, orp) and np.array_equal(ci_h, oci)   # integer work: bit-exact
    out, lse = P.gpu_forward(wl, qd, kd, vd, rp_h, ci_h)
    err, lerr = P.compare_rows(wl, out, lse, q, k, v, orp, oci, np.arange(rows))
    assert err <= P.TOL["bf16"] and lerr <= P.LSE_TOL["bf16"]
    o = out.float().cpu().reshape(rows, 64, -1)
    assert torch.all(o[[0, 7, rows - 1]] == 0)
    l = lse.cpu().reshape(rows, 64)
    assert torch.all(torch.isneginf(l[[0, 7, rows - 1]]))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_forward_skips_out_of_order_and_out_of_range_columns(dtype):
    """Both dtypes skip entries that are out of range, repeated or below the row's last
    accepted column: the output over the polluted list equals, bit for bit, the output
    over the clean one."""
    wl = small_workload("order", 2, 128 if dtype == "bf16" else 64, (2, 2, 4), dtype, seed=13)
    q, k, v, _ = make_inputs(wl, "B" if dtype == "bf16" else "A")
    qd, kd, vd = P.to_device(q, k, v)
    nB = wl.blocks
    rows = wl.heads * nB
    rng = np.random.default_rng(2)
    mask = rng.random((rows, nB)) < 0.5
    mask[:, 0] = True
    orp, oci = oracle.csr_from_mask(mask)
    out_a, lse_a = P.gpu_forward(wl, qd, kd, vd, orp, oci)
    err, lerr = P.compare_rows(wl, out_a, lse_a, q, k, v, orp, oci, np.arange(rows))
    assert err <= P.TOL[dtype] and lerr <= P.LSE_TOL[dtype]
    # entries out of range, repeated or below the previous entry are skipped
    rp2 = [0]
    ci2 = []
    for r in range(rows):
        seg = oci[orp[r]:orp[r + 1]].tolist()
        ci2 += [-1] + seg[:1] + seg[:1] + seg[1:] + [seg[0], nB + 3]
        rp2.append(len(ci2))
    out_c, lse_c = P.gpu_forward(wl, qd, kd, vd, np.array(rp2), np.array(ci2))
    assert torch.equal(out_c, out_a) and torch.equal(lse_c, lse_a)


def test_long_rows_are_split_and_merged():
    """Rows far longer than the rest are cut into pieces merged by log-sum-exp weights
    (pieces of at least 64 tiles, so rows of 105 blocks split in two).  An odd block
    count leaves the last pair of each head with a single row."""
    wl = small_workload("split", 2, 128, (7, 3, 5), "bf16", seed=23)
    q, k, v, _ = make_inputs(wl, "B")
    qd, kd, vd = P.to_device(q, k, v)
    nB = wl.blocks
    assert nB == 105
    rows = wl.heads * nB
    rng = np.random.default_rng(3)
    mask = np.zeros((rows, nB), dtype=bool)
    mask[np.arange(rows), np.arange(rows) % nB] = True
    mask[np.arange(rows), rng.integers(0, nB, rows)] = True
    long_rows = [0, 1, 50, nB - 1, nB + 51, 2 * nB - 1]
    mask[long_rows] = rng.random((len(long_rows), nB)) < 0.97
    orp, oci = oracle.csr_from_mask(mask)
    out, lse = P.gpu_forward(wl, qd, kd, vd, orp, oci)
    err, lerr = P.compare_rows(wl, out, lse, q, k, v, orp, oci, np.arange(rows))
    assert err <= P.TOL["bf16"] and lerr <= P.LSE_TOL["bf16"]
    # repeated, descending and out-of-range entries every few positions of the long rows
    # (so that they straddle the piece boundaries) are skipped as in a whole-row walk
    rp2, ci2 = [0], []
    for r in range(rows):
        seg = oci[orp[r]:orp[r + 1]].tolist()
        if r in long_rows:
            junk = []
            for n, cc in enumerate(seg):
                junk.append(cc)
                if n % 7 == 3:
                    junk += [cc, max(cc - 3, 0), -2, nB + 7]
            seg = junk
        ci2 += seg
        rp2.append(len(ci2))
    out_c, lse_c = P.gpu_forward(wl, qd, kd, vd, np.array(rp2), np.array(ci2))
    err, lerr = P.compare_rows(wl, out_c, lse_c, q, k, v, orp, oci, np.arange(rows))
    assert err <= P.TOL["bf16"] and lerr <= P.LSE_TOL["bf16"]


def test_long_rows_and_last_round_pieces_together():
    """1,024 pairs (two rounds of 512 resident workgroups): rows of 64-140 tiles, so
    the last 384 pairs in dispatch order are cut into quarter pieces, and a few rows
    of 480 tiles, cut as long rows (the per-workgroup share is ~240 tiles).  Long
    rows, rows of last-round pairs and random rows are compared with the oracle."""
    wl = small_workload("rounds", 4, 128, (8, 8, 8), "bf16", seed=31)
    q, k, v, _ = make_inputs(wl, "A")
    qd, kd, vd = P.to_device(q, k, v)
    nB = wl.blocks
    assert nB == 512 and wl.heads * nB // 2 == 1024
    rows = wl.heads * nB
    rng = np.random.default_rng(11)
    lens = rng.integers(64, 141, rows)
    long_rows = np.array([3, 700, 1301, 2047])
    lens[long_rows] = 480
    mask = np.zeros((rows, nB), dtype=bool)
    for r in range(rows):
        mask[r, rng.choice(nB, size=int(lens[r]), replace=False)] = True
    orp, oci = oracle.csr_from_mask(mask)
    out, lse = P.gpu_forward(wl, qd, kd, vd, orp, oci)
    tail = P.last_round_rows(wl)
    assert len(tail) == 12
    check = np.unique(np.concatenate([long_rows, long_rows ^ 1, tail, rng.choice(rows, 8, replace=False)]))
    err, lerr = P.compare_rows(wl, out, lse, q, k, v, orp, oci, check)
    assert err <= P.TOL["bf16"] and lerr <= P.LSE_TOL["bf16"]


def test_backward_long_rows_and_last_round_pieces():
    """The backward on 1,024 pairs with long rows: both passes cut long pairs and the
    last round into pieces whose partial rows a merge adds.  dO is nonzero only on
    sampled rows (long rows, rows of last-round pairs, random rows), so every gradient
    entry comes from them, and the oracle computes all of dQ, dK, dV from those rows."""
    wl = small_workload("bwd_rounds", 4, 128, (8, 8, 8), "bf16", seed=37)
    q, k, v, _ = make_inputs(wl, "A")
    qd, kd, vd = P.to_device(q, k, v)
    nB = wl.blocks
    rows = wl.heads * nB
    rng = np.random.default_rng(13)
    lens = rng.integers(64, 141, rows)
    long_rows = np.array([5, 900, 1500, 2046])
    lens[long_rows] = 480
    mask = np.zeros((rows, nB), dtype=bool)
    for r in range(rows):
        mask[r, rng.choice(nB, size=int(lens[r]), replace=False)] = True
    orp, oci = oracle.csr_from_mask(mask)
    _, lse = P.gpu_forward(wl, qd, kd, vd, orp, oci)
    q32, k32, v32 = (t.float().numpy() for t in (q, k, v))
    sample = np.unique(np.concatenate([long_rows, P.last_round_rows(wl), rng.choice(rows, 4, replace=False)]))
    P.backward_sampled(wl, P.shape_for(wl), qd, kd, vd, lse, q32, k32, v32, orp, oci, sample)


@pytest.mark.parametrize("dtype,d,grid,tile", [("bf16", 128, (3, 16, 24), (1, 8, 8)),
                                                 ("f32", 64, (4, 8, 16), (2, 4, 8)),
                                                 ("bf16", 64, (2, 32, 8), (1, 8, 8))])
def test_token_reorder_matches_oracle(dtype, d, grid, tile):
    """Raster <-> tile-major reordering is a permutation: bit-exact against the oracle."""
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    gen = torch.Generator().manual_seed(6)
    x = torch.randn((2, 3, grid[0] * grid[1] * grid[2], d), generator=gen).to(tdt)
    shape = B.make_shape(2, 3, d, grid, dtype, 0.0, tile)
    xd = x.cuda()
    y = B.sparse_attn_to_tiles(shape, xd)
    z = B.sparse_attn_from_tiles(shape, y)
    torch.cuda.synchronize()
    ref = oracle.to_tiles(x.float(), grid, tile)
    assert np.array_equal(y.float().cpu().numpy(), ref)
    assert torch.equal(z.cpu(), x)


RASTER = [
    # name, heads, d, block grid, dtype, thr, window, reading, head-thr range
    ("bf16_d128", 2, 128, (3, 5, 7), "bf16", 0.85, (-1, -1, -1), "A", None),
    ("f32_d64_window", 2, 64, (2, 3, 5), "f32", 0.9, (1, 1, 1), "B", None),
    ("bf16_d64_window", 3, 64, (2, 4, 6), "bf16", 0.7, (1, 1, 1), "B", None),
    ("bf16_d128_756_headthr", 2, 128, (3, 12, 21), "bf16", 0.8, (-1, -1, -1), "A", (0.6, 0.9)),
]


@pytest.mark.parametrize("case", RASTER, ids=[c[0] for c in RASTER])
def test_raster_selection(case):
    """The selection on raster inputs: tile-major copies bit-equal to the inputs of the
    tiled path, and the block list against the oracle (differences only at the CDF
    boundary)."""
    name, H, d, bg, dt, thr, win, reading, hr = case
    wl = small_workload(name, H, d, bg, dt, threshold=thr, window=win, head_threshold_range=hr, seed=23)
    print(f"\n[case] raster selection {name} blocks={wl.blocks}", flush=True)
    q, k, _, thr_h = make_inputs(wl, reading)
    qd, kd = P.to_device(q, k)
    shape = P.shape_for(wl)
    qr, kr = B.sparse_attn_from_tiles(shape, qd), B.sparse_attn_from_tiles(shape, kd)
    head_thr = None if hr is None else [float(x) for x in thr_h]
    rp, ci, qt, kt = B.sparse_attn_select_raster(shape, qr, kr, threshold=float(np.float32(wl.threshold)),
                                                 head_thresholds=head_thr, window=win)
    torch.cuda.synchronize()
    assert torch.equal(qt, qd) and torch.equal(kt, kd)
    rp_h = rp.cpu().numpy().astype(np.int64)
    gmask = P.check_csr(rp_h, ci[:int(rp_h[-1])].cpu().numpy(), wl.blocks)
    qbar, kbar, keep, band = P.oracle_select_full(wl, q, k, thr_h, count_band=True)
    rep = P.compare_masks(gmask, keep, qbar, kbar, wl, thr_h, band=band)
    P.record_masks(f"raster_{name}", rep)
    assert P.mask_ok(rep), P.fmt(rep)


def test_full_csr_is_the_dense_block_list():
    """The dense block list equals the oracle's CSR of an all-true mask (integer work:
    bit-exact), and attention over it is dense attention."""
    wl = small_workload("full", 2, 64, (2, 3, 3), "bf16", seed=29)
    shape = P.shape_for(wl)
    rows, nB = wl.heads * wl.blocks, wl.blocks
    rp, ci = B.sparse_attn_full_csr(shape)
    torch.cuda.synchronize()
    orp, oci = oracle.csr_from_mask(np.ones((rows, nB), dtype=bool))
    rp_h = rp.cpu().numpy().astype(np.int64)
    assert np.array_equal(rp_h, orp) and np.array_equal(ci[:int(rp_h[-1])].cpu().numpy(), oci)
    q, k, v, _ = make_inputs(wl, "A")
    qd, kd, vd = P.to_device(q, k, v)
    out, lse = P.gpu_forward(wl, qd, kd, vd, rp_h, ci[:int(rp_h[-1])].cpu().numpy())
    err, lerr = P.compare_rows(wl, out, lse, q, k, v, orp, oci, np.arange(rows))
    assert err <= P.TOL["bf16"] and lerr <= P.LSE_TOL["bf16"]


def _random_offsets(rng, n):
    """-ln(pi) for inclusion probabilities spread over (0.02, 1]: offsets from 0 to ~3.9."""
    return -np.log(rng.uniform(0.02, 1.0, n))


@pytest.mark.parametrize("d,grid,reading,dt", [(128, (3, 4, 5), "A", "bf16"), (64, (2, 3, 5), "B", "bf16"),
                                               (64, (2, 3, 5), "A", "f32"), (128, (3, 4, 5), "B", "f32")])
def test_biased_forward_matches_oracle(d, grid, reading, dt):
    """Attention with a logit offset per block-list entry against the oracle with the
    same offsets, on a random block list with empty rows (bf16 and fp32)."""
    wl = small_workload("bias", 2, d, grid, dt, seed=51)
    q, k, v, _ = make_inputs(wl, reading)
    qd, kd, vd = P.to_device(q, k, v)
    rows, nB = wl.heads * wl.blocks, wl.blocks
    rng = np.random.default_rng(52)
    mask = rng.random((rows, nB)) < 0.4
    mask[[3, nB + 5]] = False
    orp, oci = oracle.csr_from_mask(mask)
    bias = _random_offsets(rng, len(oci)).astype(np.float32)
    out, lse = P.gpu_forward_biased(wl, qd, kd, vd, orp, oci, bias)
    err, lerr = P.compare_rows(wl, out, lse, q, k, v, orp, oci, np.arange(rows), bias=bias.astype(np.float64))
    print(f"biased forward {dt} d={d}: max|err| {err:.3e} lse {lerr:.3e}", flush=True)
    tol, ltol = P.forward_tols(dt, reading)
    assert err <= tol and lerr <= ltol
    # zero offsets against the plain kernel: the offset path keeps its running max in
    # log2 units, so the lazy max may move at another tile and P round differently in
    # bf16; both stay within the output bound of each other
    out0, lse0 = P.gpu_forward_biased(wl, qd, kd, vd, orp, oci, np.zeros(len(oci), np.float32))
    out1, lse1 = P.gpu_forward(wl, qd, kd, vd, orp, oci)
    assert float((out0.float() - out1.float()).abs().max()) <= P.TOL[dt]
    assert torch.equal(torch.isinf(lse0), torch.isinf(lse1))
    fin = torch.isfinite(lse1)
    assert float((lse0[fin] - lse1[fin]).abs().max()) <= P.LSE_TOL[dt]


def test_biased_forward_split_rows():
    """Offsets on rows long enough to be split into pieces and merged."""
    wl = small_workload("biassplit", 2, 128, (7, 3, 5), "bf16", seed=53)
    q, k, v, _ = make_inputs(wl, "A")
    qd, kd, vd = P.to_device(q, k, v)
    nB = wl.blocks
    rows = wl.heads * nB
    rng = np.random.default_rng(54)
    mask = np.zeros((rows, nB), dtype=bool)
    mask[np.arange(rows), np.arange(rows) % nB] = True
    long_rows = [0, 1, 50, nB + 51]
    mask[long_rows] = rng.random((len(long_rows), nB)) < 0.97
    orp, oci = oracle.csr_from_mask(mask)
    bias = _random_offsets(rng, len(oci)).astype(np.float32)
    out, lse = P.gpu_forward_biased(wl, qd, kd, vd, orp, oci, bias)
    err, lerr = P.compare_rows(wl, out, lse, q, k, v, orp, oci, np.arange(rows), bias=bias.astype(np.float64))
    assert err <= P.TOL["bf16"] and lerr <= P.LSE_TOL["bf16"]


@pytest.mark.parametrize("d,grid,budget,reading,dt", [(128, (3, 4, 5), 6.5, "A", "bf16"),
                                                      (64, (4, 4, 5), 3.0, "B", "bf16"),
                                                      (128, (2, 8, 18), 40.0, "A", "bf16"),
                                                      (64, (3, 4, 5), 6.5, "A", "f32"),
                                                      (128, (2, 8, 18), 40.0, "B", "f32")])
def test_sip_selection_matches_oracle(d, grid, budget, reading, dt):
    """Sampled block lists and their offsets against the oracle (differences only where
    a block's uniform lies within the stated band of its inclusion probability); bf16
    and fp32 inputs."""
    from oracle import sip
    wl = small_workload("sip", 2, d, grid, dt, seed=55)
    q, k, _, _ = make_inputs(wl, reading)
    qd, kd = P.to_device(q, k)
    shape = P.shape_for(wl)
    rp, ci, cb = B.sparse_attn_select_sip(shape, qd, kd, budget, seed=1234)
    torch.cuda.synchronize()
    rp_h = rp.cpu().numpy().astype(np.int64)
    nnz = int(rp_h[-1])
    keep, _, _, _, pi, u = sip.select_sip(q, k, wl.heads, budget, seed=1234)
    ndiff, unexcused, berr = P.compare_sip(rp_h, ci[:nnz].cpu().numpy(), cb[:nnz].cpu().numpy(), keep, pi, u,
                                           wl.blocks)
    print(f"sip d={d} nB={wl.blocks} budget={budget}: kept {nnz} (oracle {int(keep.sum())}), "
          f"differing {ndiff}, unexcused {unexcused}, max offset err {berr:.2e}", flush=True)
    assert unexcused == 0 and berr <= P.SIP_BIAS_TOL


def test_sip_budget_of_all_blocks_keeps_everything():
    wl = small_workload("sipall", 1, 64, (2, 3, 3), "bf16", seed=57)
    q, k, _, _ = make_inputs(wl, "A")
    qd, kd = P.to_device(q, k)
    rp, ci, cb = B.sparse_attn_select_sip(P.shape_for(wl), qd, kd, float(wl.blocks), seed=3)
    torch.cuda.synchronize()
    nB, rows = wl.blocks, wl.heads * wl.blocks
    assert np.array_equal(rp.cpu().numpy(), np.arange(rows + 1) * nB)
    assert np.array_equal(ci[:rows * nB].cpu().numpy(), np.tile(np.arange(nB), rows))
    assert torch.all(cb[:rows * nB] == 0)


@pytest.mark.parametrize("d,grid,thr,reading,dt", [(128, (3, 4, 5), 0.8, "A", "bf16"), (64, (2, 3, 5), 0.9, "B", "bf16"),
                                                  (128, (2, 8, 18), 0.7, "A", "bf16"), (64, (3, 4, 5), 0.8, "A", "f32"),
                                                  (128, (2, 8, 18), 0.7, "B", "f32")])
def test_ibcs_selection_matches_oracle(d, grid, thr, reading, dt):
    """The clustering selector against the oracle: block lists equal except at the CDF
    boundary, and pairs with near-tied k-means assignments checked for validity; bf16
    and fp32 queries."""
    from oracle import ibcs
    wl = small_workload("ibcs", 2, d, grid, dt, threshold=thr, seed=61)
    q, k, _, _ = make_inputs(wl, reading)
    qd, kd = P.to_device(q, k)
    rp, ci = B.sparse_attn_select_ibcs(P.shape_for(wl), qd, kd, threshold=thr)
    torch.cuda.synchronize()
    rp_h = rp.cpu().numpy().astype(np.int64)
    gmask = P.check_csr(rp_h, ci[:int(rp_h[-1])].cpu().numpy(), wl.blocks)
    keep, _, _, pt, gaps = ibcs.select_ibcs(q.float().numpy(), k.float().numpy(), wl.heads, thr)
    nB = wl.blocks
    pair_of_row = (np.arange(wl.heads * nB) % nB) // 2 + (np.arange(wl.heads * nB) // nB) * ((nB + 1) // 2)
    skip = gaps.reshape(-1)[pair_of_row] < P.IBCS_GAP
    ndiff, nexc, nunx = P.compare_cdf_rows(gmask, keep, pt, np.full(len(keep), thr), skip)
    near_diff = int((gmask[skip] != keep[skip]).sum())
    # validity on every row: the kept mass reaches the threshold (on the oracle's p~)
    mass = (pt * gmask).sum(axis=1)
    print(f"ibcs d={d} nB={nB}: kept {int(gmask.sum())} (oracle {int(keep.sum())}), differing {ndiff}, "
          f"excused {nexc}, unexcused {nunx}, near-tie rows {int(skip.sum())} (differing there {near_diff})", flush=True)
    assert nunx == 0
    # the kept mass on the oracle's p~: within the R1 band of the threshold where the
    # clustering matches; a near-tie pair may cluster differently on the GPU, which moves
    # p~ itself, so only a looser 1e-3 holds there
    assert np.all(mass[~skip] >= thr - 1e-4) and np.all(mass[skip] >= thr - 1e-3)
    # both blocks of a pair share the row
    for r in range(0, wl.heads * nB - 1):
        if (r % nB) % 2 == 0 and (r % nB) + 1 < nB:
            assert np.array_equal(gmask[r], gmask[r + 1])


def test_ibcs_runs_four_kmeans_rounds():
    """The kernel's k-means round count, pinned through the block list.  Every pair of
    query blocks holds the hand-derived chain of the k-means golden case (shifted by
    -9 along the first axis, so that the two moving centroids take opposite signs)
    and its six frozen groups along the second axis, where the keys are zero (they add
    a uniform share).  Key block j is c_j along the first axis, c_j distinct multiples
    of 1/8.  The mixture's order then depends on where the two centroids sit, and on
    the oracle the block lists after 1, 2, 3, 5 and 6 rounds all differ from the one
    after 4; the GPU's must equal the 4-round list exactly (every cumulative mass is
    more than 1e-2 from the threshold and neighbouring p~ differ by > 7e-4 relative,
    far above the kernel's rounding)."""
    from oracle import ibcs
    from .test_oracle_pins import _kmeans_chain_golden
    x, _ = _kmeans_chain_golden()
    nB, d, thr, scale = 32, 128, 0.5, 0.25
    q = np.zeros((1, 1, nB * 64, d), dtype=np.float32)
    for p in range(nB // 2):
        q[0, 0, 128 * p:128 * p + 32, 0] = x[:32, 0] - 9.0
        q[0, 0, 128 * p + 32:128 * p + 128, 1] = x[32:, 0]
    c = (np.arange(nB) - 15.5) / 8.0
    np.random.default_rng(5).shuffle(c)
    k = np.zeros((1, 1, nB * 64, d), dtype=np.float32)
    k[0, 0, :, 0] = np.repeat(c, 64)
    masks = {it: ibcs.select_ibcs(q, k, 1, thr, scale=scale, iters=it)[0] for it in (1, 2, 3, 4, 5, 6)}
    assert all((masks[it] != masks[4]).any() for it in (1, 2, 3, 5, 6))
    shape = B.make_shape(1, 1, d, (1, 32, 64), "bf16", scale)
    qd = torch.as_tensor(q).to(torch.bfloat16).cuda()
    kd = torch.as_tensor(k).to(torch.bfloat16).cuda()
    rp, ci = B.sparse_attn_select_ibcs(shape, qd, kd, threshold=thr)
    torch.cuda.synchronize()
    rp_h = rp.cpu().numpy().astype(np.int64)
    gmask = P.check_csr(rp_h, ci[:int(rp_h[-1])].cpu().numpy(), nB)
    assert np.array_equal(gmask, masks[4])


def _backward_case(wl, reading, mask=None, seed=0):
    q, k, v, _ = make_inputs(wl, reading)
    qd, kd, vd = P.to_device(q, k, v)
    shape = P.shape_for(wl)
    rows, nB = wl.heads * wl.blocks, wl.blocks
    if mask is None:
        qbar, kbar = oracle.pool(q), oracle.pool(k)
        mask = oracle.select_rows(qbar, kbar, wl.heads, wl.block_grid, float(wl.threshold)) != 0
    orp, oci = oracle.csr_from_mask(mask)
    out, lse = P.gpu_forward(wl, qd, kd, vd, orp, oci)
    gen = torch.Generator().manual_seed(seed)
    g = torch.randn(q.shape, generator=gen).to(torch.bfloat16)
    return q, k, v, qd, kd, vd, out, lse, g, shape, orp, oci


def _rel_err(got, ref):
    got = got.float().cpu().numpy().astype(np.float64)
    return float(np.abs(got - ref).max() / max(np.abs(ref).max(), 1e-30))


@pytest.mark.parametrize("d,grid,thr,reading,seed", [(128, (3, 4, 5), 0.8, "A", 31), (64, (2, 3, 5), 0.9, "B", 37)])
def test_backward_matches_oracle(d, grid, thr, reading, seed):
    """dQ, dK, dV against the fp64 oracle under the same block list; the block count
    is odd, so the last pair of each head has one block."""
    wl = small_workload("bwd", 2, d, grid, "bf16", threshold=thr, seed=seed)
    q, k, v, qd, kd, vd, out, lse, g, shape, orp, oci = _backward_case(wl, reading, seed=seed)
    rpd = torch.as_tensor(orp.astype(np.int32)).cuda()
    cid = torch.as_tensor(oci).cuda()
    dq, dk, dv = B.sparse_attn_backward(shape, qd, kd, vd, out, lse, g.cuda(), rpd, cid)
    torch.cuda.synchronize()
    rq, rk, rv = oracle.attention_backward(q, k, v, g, orp, oci)
    errs = [_rel_err(x, r) for x, r in ((dq, rq), (dk, rk), (dv, rv))]
    print(f"backward rel err dq {errs[0]:.3e} dk {errs[1]:.3e} dv {errs[2]:.3e}", flush=True)
    assert max(errs[:2]) <= P.BWD_TOL_DQK and errs[2] <= P.BWD_TOL_DV
    # Same stored output on both sides (the oracle's forward, rounded to bf16): what
    # is left is the kernels' own rounding of P and dS.
    o_ref, _ = oracle.attention_rows(q, k, v, orp, oci, np.arange(wl.heads * wl.blocks))
    o_bf = torch.as_tensor(o_ref.reshape(q.shape)).to(torch.bfloat16)
    dq, dk, dv = B.sparse_attn_backward(shape, qd, kd, vd, o_bf.cuda(), lse, g.cuda(), rpd, cid)
    torch.cuda.synchronize()
    rq, rk, rv = oracle.attention_backward(q, k, v, g, orp, oci, out=o_bf.float())
    errs = [_rel_err(x, r) for x, r in ((dq, rq), (dk, rk), (dv, rv))]
    print(f"backward (same O) rel err dq {errs[0]:.3e} dk {errs[1]:.3e} dv {errs[2]:.3e}", flush=True)
    assert max(errs[:2]) <= P.BWD_TOL_DQK and errs[2] <= P.BWD_TOL_DV


def test_backward_empty_rows_unused_keys_and_skipped_entries():
    """Empty query rows get dQ = 0, key blocks nobody keeps get dK = dV = 0, and
    repeated, descending or out-of-range entries change nothing (bit-exact)."""
    wl = small_workload("bwd2", 2, 128, (3, 3, 3), "bf16", seed=41)
    nB = wl.blocks
    rows = wl.heads * nB
    rng = np.random.default_rng(6)
    mask = rng.random((rows, nB)) < 0.5
    mask[:, 4] = False                               # key block 4: unused
    mask[[0, nB + 7]] = False                        # empty rows
    mask[1, :] = np.arange(nB) != 4
    q, k, v, qd, kd, vd, out, lse, g, shape, orp, oci = _backward_case(wl, "A", mask=mask, seed=43)
    gd = g.cuda()
    rpd = torch.as_tensor(orp.astype(np.int32)).cuda()
    cid = torch.as_tensor(oci).cuda()
    dq, dk, dv = B.sparse_attn_backward(shape, qd, kd, vd, out, lse, gd, rpd, cid)
    rq, rk, rv = oracle.attention_backward(q, k, v, g, orp, oci)
    assert max(_rel_err(dq, rq), _rel_err(dk, rk)) <= P.BWD_TOL_DQK and _rel_err(dv, rv) <= P.BWD_TOL_DV
    dqh = dq.float().cpu().reshape(rows, 64, -1)
    assert torch.all(dqh[[0, nB + 7]] == 0)
    dkh, dvh = dk.float().cpu().reshape(rows, 64, -1), dv.float().cpu().reshape(rows, 64, -1)
    assert torch.all(dkh[[4, nB + 4]] == 0) and torch.all(dvh[[4, nB + 4]] == 0)
    rp2, ci2 = [0], []
    for r in range(rows):
        seg = oci[orp[r]:orp[r + 1]].tolist()
        ci2 += [-3] + seg[:1] + seg + [nB + 1] + seg[:1]
        rp2.append(len(ci2))
    rpd2 = torch.as_tensor(np.array(rp2, dtype=np.int32)).cuda()
    cid2 = torch.as_tensor(np.array(ci2, dtype=np.int32)).cuda()
    dq2, dk2, dv2 = B.sparse_attn_backward(shape, qd, kd, vd, out, lse, gd, rpd2, cid2)
    torch.cuda.synchronize()
    assert torch.equal(dq2, dq) and torch.equal(dk2, dk) and torch.equal(dv2, dv)


@pytest.mark.parametrize("name,d,grid,thr,reading", [("bf16_d128_2x12x20", 128, (2, 12, 20), 0.8, "A"),
                                                      ("bf16_d64_3x13x11_B", 64, (3, 13, 11), 0.9, "B")])
def test_backward_partial_tiles(name, d, grid, thr, reading):
    """Partial tiles in the backward: dQ, dK, dV against the oracle with the same token
    validity, junk in every padding slot of Q, K, V and dO; padding slots get exact
    zeros in all three gradients."""
    wl = small_workload("bwd_partial_" + name, 2, d, (0, 0, 0), "bf16", threshold=thr, seed=73, grid=grid)
    assert wl.partial
    print(f"\n[case] backward partial tiles {name} blocks={wl.blocks} slots={wl.slots}", flush=True)
    q, k, v, _ = make_inputs(wl, reading)
    gen = torch.Generator().manual_seed(74)
    g = torch.randn(q.shape, generator=gen).to(torch.bfloat16)
    q, k, v, g = _junk_padding(wl, q, k, v, g)
    valid = P.valid_of(wl)
    qd, kd, vd = P.to_device(q, k, v)
    shape = P.shape_for(wl)
    qbar, kbar = oracle.pool(q, valid=valid), oracle.pool(k, valid=valid)
    mask = oracle.select_rows(qbar, kbar, wl.heads, wl.block_grid, float(wl.threshold)) != 0
    orp, oci = oracle.csr_from_mask(mask)
    out, lse = P.gpu_forward(wl, qd, kd, vd, orp, oci)
    rpd = torch.as_tensor(orp.astype(np.int32)).cuda()
    cid = torch.as_tensor(oci).cuda()
    dq, dk, dv = B.sparse_attn_backward(shape, qd, kd, vd, out, lse, g.cuda(), rpd, cid)
    torch.cuda.synchronize()
    rq, rk, rv = oracle.attention_backward(q, k, v, g, orp, oci, valid=valid)
    errs = [_rel_err(x, r) for x, r in ((dq, rq), (dk, rk), (dv, rv))]
    print(f"backward partial rel err dq {errs[0]:.3e} dk {errs[1]:.3e} dv {errs[2]:.3e}", flush=True)
    assert max(errs[:2]) <= P.BWD_TOL_DQK and errs[2] <= P.BWD_TOL_DV
    vt = torch.as_tensor(valid)
    for gr in (dq, dk, dv):
        assert torch.all(gr.cpu()[..., ~vt, :] == 0)


@pytest.mark.parametrize("name,d,grid,bgrid,thr,reading", [
    ("f32_d64", 64, None, (2, 3, 5), 0.9, "A"),
    ("f32_d128_B", 128, None, (3, 4, 3), 0.8, "B"),
    ("f32_d64_partial_3x13x11", 64, (3, 13, 11), (0, 0, 0), 0.85, "A"),
])
def test_backward_f32(name, d, grid, bgrid, thr, reading):
    """The fp32 backward (fp32 MFMA, one workgroup per block) against the oracle on the
    same block list: whole tiles at d = 64 and 128 (odd block counts), and a grid with
    partial tiles (junk in every padding slot; exact zeros there)."""
    wl = small_workload("bwd_f32_" + name, 2, d, bgrid, "f32", threshold=thr, seed=75, grid=grid)
    print(f"\n[case] fp32 backward {name} blocks={wl.blocks} slots={wl.slots}", flush=True)
    q, k, v, _ = make_inputs(wl, reading)
    gen = torch.Generator().manual_seed(76)
    g = torch.randn(q.shape, generator=gen, dtype=torch.float32)
    valid = P.valid_of(wl)
    if valid is not None:
        q, k, v, g = _junk_padding(wl, q, k, v, g)
    qd, kd, vd = P.to_device(q, k, v)
    shape = P.shape_for(wl)
    qbar, kbar = oracle.pool(q, valid=valid), oracle.pool(k, valid=valid)
    mask = oracle.select_rows(qbar, kbar, wl.heads, wl.block_grid, float(wl.threshold)) != 0
    orp, oci = oracle.csr_from_mask(mask)
    out, lse = P.gpu_forward(wl, qd, kd, vd, orp, oci)
    rpd = torch.as_tensor(orp.astype(np.int32)).cuda()
    cid = torch.as_tensor(oci).cuda()
    dq, dk, dv = B.sparse_attn_backward(shape, qd, kd, vd, out, lse, g.cuda(), rpd, cid)
    torch.cuda.synchronize()
    rq, rk, rv = oracle.attention_backward(q, k, v, g, orp, oci, valid=valid)
    errs = [_rel_err(x, r) for x, r in ((dq, rq), (dk, rk), (dv, rv))]
    print(f"fp32 backward rel err dq {errs[0]:.3e} dk {errs[1]:.3e} dv {errs[2]:.3e}", flush=True)
    assert max(errs) <= P.BWD_TOL_F32
    if valid is not None:
        vt = torch.as_tensor(valid)
        for gr in (dq, dk, dv):
            assert torch.all(gr.cpu()[..., ~vt, :] == 0)


def test_deterministic_and_no_nan():
    wl = small_workload("det", 3, 128, (3, 4, 5), "bf16", threshold=0.8, window=(1, 1, 1), seed=17)
    q, k, v, thr = make_inputs(wl, "A")
    qd, kd, vd = P.to_device(q, k, v)
    shape = P.shape_for(wl)
    bufs = B.alloc_buffers(shape)
    bufs.col_idx.fill_(-7)
    results = []
    for _ in range(2):
        rp, ci = B.sparse_attn_select(shape, qd, kd, threshold=wl.threshold, window=wl.window, buffers=bufs)
        rp = rp.clone()
        ci = ci[:int(rp[-1].item())].clone()
        out = torch.full_like(qd, float("nan"))
        lse = torch.full(qd.shape[:3], float("nan"), device="cuda")
        B.sparse_attn_forward(shape, qd, kd, vd, rp, ci, out=out, lse=lse)
        torch.cuda.synchronize()
        results.append((rp.cpu(), ci.cpu(), out.cpu(), lse.cpu()))
    for a, b in zip(*results):
        assert torch.equal(a, b)
    assert not torch.isnan(results[0][2].float()).any() and not torch.isnan(results[0][3]).any()


def test_nondefault_scale():
    wl = small_workload("scale", 2, 64, (2, 2, 3), "f32", threshold=0.75, seed=19)
    q, k, v, thr = make_inputs(wl, "A")
    qd, kd, vd = P.to_device(q, k, v)
    shape = B.make_shape(1, wl.heads, wl.head_dim, wl.grid, "f32", scale=0.5)
    rp, ci = B.sparse_attn_select(shape, qd, kd, threshold=0.75)
    torch.cuda.synchronize()
    rp_h = rp.cpu().numpy().astype(np.int64)
    gmask = P.check_csr(rp_h, ci[:int(rp_h[-1])].cpu().numpy(), wl.blocks)
    qbar, kbar = oracle.pool(q), oracle.pool(k)
    keep = oracle.select_rows(qbar, kbar, wl.heads, wl.block_grid, 0.75, scale=0.5)
    assert (gmask == (keep != 0)).mean() > 0.999
    orp, oci = oracle.csr_from_mask(keep != 0)
    rpd = torch.as_tensor(orp.astype(np.int32)).cuda()
    cid = torch.as_tensor(oci).cuda()
    out, lse = B.sparse_attn_forward(shape, qd, kd, vd, rpd, cid, want_lse=True)
    torch.cuda.synchronize()
    ref, ref_lse = oracle.attention_rows(q, k, v, orp, oci, np.arange(wl.heads * wl.blocks), scale=0.5)
    got = out.cpu().reshape(-1, 64, wl.head_dim).numpy()
    assert np.abs(got - ref).max() <= P.TOL["f32"]
    assert np.abs(lse.cpu().reshape(-1, 64).numpy() - ref_lse).max() <= P.LSE_TOL["f32"]


def test_tiny_workload_full():
    wl = WORKLOADS["tiny_f32"]
    q, k, v, thr = make_inputs(wl, "A")
    qd, kd, vd = P.to_device(q, k, v)
    rp, ci = P.gpu_select(wl, qd, kd, thr)
    gmask = P.check_csr(rp, ci, wl.blocks)
    qbar, kbar, keep, band = P.oracle_select_full(wl, q, k, thr, count_band=True)
    rep = P.compare_masks(gmask, keep, qbar, kbar, wl, thr, band=band)
    P.record_masks("tiny_f32_A", rep)
    assert P.mask_ok(rep), P.fmt(rep)
    orp, oci = oracle.csr_from_mask(keep != 0)
    out, lse = P.gpu_forward(wl, qd, kd, vd, orp, oci)
    err, lerr = P.compare_rows(wl, out, lse, q, k, v, orp, oci, np.arange(wl.blocks))
    print(f"tiny forward err={err:.3e} lse={lerr:.3e}", flush=True)
    assert err <= P.TOL["f32"] and lerr <= P.LSE_TOL["f32"]


@pytest.mark.parametrize("grid,tile,heads,r0,gamma,lam", [
    ((4, 16, 24), (1, 8, 8), 2, 2.5, 0.6, 0),
    ((6, 24, 16), (1, 8, 8), 1, 3.0, 0.5, 2),
    ((20, 32, 48), (1, 8, 8), 3, 4.0, 0.7, 3),      # the 480p block grid
    ((32, 48, 80), (1, 8, 8), 1, 6.0, 0.8, 4),      # the HunyuanVideo-like block grid
    ((8, 16, 16), (2, 4, 8), 2, 0.5, 0.9, 1),       # r0 < 1: own block and every frame's co-located one
])
def test_radial_csr_matches_oracle(grid, tile, heads, r0, gamma, lam):
    """DynamicRad's radial window: bit-exact against the oracle's mask, for every head."""
    from oracle import radial
    shape = B.make_shape(1, heads, 128, grid, "bf16", 0.0, tile)
    rp, ci = B.sparse_attn_radial_csr(shape, r0, gamma, lam)
    torch.cuda.synchronize()
    block_grid = (grid[0] // tile[0], grid[1] // tile[1], grid[2] // tile[2])
    m = radial.radial_mask(block_grid, r0, gamma, lam)
    orp, oci = oracle.csr_from_mask(np.tile(m, (heads, 1)))
    nnz = int(orp[-1])
    assert np.array_equal(rp.cpu().numpy(), orp.astype(np.int32))
    assert np.array_equal(ci[:nnz].cpu().numpy(), oci)


def test_lookback_give_up_is_reported(monkeypatch):
    """With the look-back's wait cut to zero polls, a row group that finds an earlier
    group's total still unpublished gives up at once.  Either no group had to wait (the
    check says OK and the block list equals the normal one) or the check reports the
    fault and row_ptr holds -1 entries: the list is never silently wrong.  Every access
    stays in bounds either way (a group that gives up writes no columns, and missing
    totals only make later offsets smaller).  A normal selection on the same workspace
    then clears the fault."""
    wl = WORKLOADS["wan13b_480p"].with_(heads=4)
    q, k, _, thr = make_inputs(wl, "A")
    qd, kd = P.to_device(q, k)
    shape = P.shape_for(wl)
    ref_rp, ref_ci = P.gpu_select(wl, qd, kd, thr)
    bufs = B.alloc_buffers(shape)
    faults = 0
    monkeypatch.setenv("SPARSE_ATTN_LOOKBACK_SPIN_CAP", "0")
    for _ in range(3):
        B.sparse_attn_select(shape, qd, kd, threshold=wl.threshold, buffers=bufs)
        st = B.sparse_attn_select_check(shape, bufs.workspace)
        rp = bufs.row_ptr.cpu().numpy().astype(np.int64)
        if st == B.SPARSE_ATTN_OK:
            assert np.array_equal(rp, ref_rp)
            assert np.array_equal(bufs.col_idx[:int(rp[-1])].cpu().numpy(), ref_ci)
        else:
            assert st == B.SPARSE_ATTN_LOOKBACK_FAULT
            assert (rp == -1).any()
            faults += 1
    print(f"give-ups reported in {faults} of 3 selections", flush=True)
    monkeypatch.delenv("SPARSE_ATTN_LOOKBACK_SPIN_CAP")
    B.sparse_attn_select(shape, qd, kd, threshold=wl.threshold, buffers=bufs)
    assert B.sparse_attn_select_check(shape, bufs.workspace) == B.SPARSE_ATTN_OK
    rp = bufs.row_ptr.cpu().numpy().astype(np.int64)
    assert np.array_equal(rp, ref_rp)



# ---------------------------------------------------------------- partial tiles
# Grids that are not a whole number of tiles: the last tile along y or x is partial,
# and its slots beyond the grid are padding (filled here with junk, which must not
# matter).

PARTIAL = [
    # name, heads, d, token grid, dtype, thr, window, reading
    ("bf16_d128_2x12x20", 2, 128, (2, 12, 20), "bf16", 0.85, (-1, -1, -1), "A"),
    ("f32_d64_3x13x11", 1, 64, (3, 13, 11), "f32", 0.9, (-1, -1, -1), "A"),
    ("bf16_d64_4x9x17_window", 2, 64, (4, 9, 17), "bf16", 0.7, (1, 1, 1), "B"),
    ("bf16_d128_5x20x36_page", 3, 128, (5, 20, 36), "bf16", 0.9, (-1, -1, -1), "page"),
]


def _junk_padding(wl, *ts):
    valid = torch.as_tensor(P.valid_of(wl))
    for t in ts:
        t[..., ~valid, :] = 7.0
    return ts


@pytest.mark.parametrize("case", PARTIAL, ids=[c[0] for c in PARTIAL])
def test_partial_tiles_select_and_forward(case):
    name, H, d, grid, dt, thr, win, reading = case
    wl = small_workload(name, H, d, (0, 0, 0), dt, threshold=thr, window=win, seed=71, grid=grid)
    assert wl.partial
    print(f"\n[case] partial tiles {name} blocks={wl.blocks} tokens={wl.tokens} slots={wl.slots}", flush=True)
    q, k, v, thr_h = make_inputs(wl, reading)
    q, k, v = _junk_padding(wl, q, k, v)
    qd, kd, vd = P.to_device(q, k, v)
    rp, ci = P.gpu_select(wl, qd, kd, thr_h)
    gmask = P.check_csr(rp, ci, wl.blocks)
    qbar, kbar, keep, band = P.oracle_select_full(wl, q, k, thr_h, count_band=True)
    rep = P.compare_masks(gmask, keep, qbar, kbar, wl, thr_h, band=band)
    P.record_masks(f"partial_{name}", rep)
    assert P.mask_ok(rep), P.fmt(rep)
    orp, oci = oracle.csr_from_mask(keep != 0)
    out, lse = P.gpu_forward(wl, qd, kd, vd, orp, oci)
    rows = np.arange(wl.heads * wl.blocks)
    err, lerr = P.compare_rows(wl, out, lse, q, k, v, orp, oci, rows)
    print(f"forward max|err|={err:.3e} lse max|err|={lerr:.3e}", flush=True)
    tol, ltol = P.forward_tols(dt, reading)
    assert err <= tol and lerr <= ltol
    valid = torch.as_tensor(P.valid_of(wl))
    assert torch.all(out.cpu()[..., ~valid, :] == 0)


@pytest.mark.parametrize("dt,d", [("bf16", 128), ("f32", 64)])
def test_partial_tiles_reorder_and_raster_selection(dt, d):
    """to_tiles / from_tiles on a grid with partial tiles are bit-exact against the
    oracle's index map (zeros in the padding slots), and the selection on raster inputs
    writes the same tile-major copies and keeps the oracle's blocks."""
    wl = small_workload("partial_raster", 2, d, (0, 0, 0), dt, threshold=0.85, seed=72, grid=(3, 11, 21))
    q, k, _, thr = make_inputs(wl, "A")
    shape = P.shape_for(wl)
    def moved(x, f):
        # the oracle's index maps move bit patterns: bf16 travels as int16 (numpy has no bf16)
        if x.dtype == torch.bfloat16:
            return torch.as_tensor(f(x.view(torch.int16), wl.grid, wl.tile)).view(torch.bfloat16)
        return torch.as_tensor(f(x, wl.grid, wl.tile))

    qr = moved(q, oracle.from_tiles).cuda()
    kr = moved(k, oracle.from_tiles).cuda()
    qt = B.sparse_attn_to_tiles(shape, qr)
    back = B.sparse_attn_from_tiles(shape, qt)
    torch.cuda.synchronize()
    assert torch.equal(qt.cpu(), moved(qr.cpu(), oracle.to_tiles))
    assert torch.equal(qt.cpu(), q) and torch.equal(back, qr)
    rp, ci, qt2, kt2 = B.sparse_attn_select_raster(shape, qr, kr, threshold=float(np.float32(wl.threshold)))
    torch.cuda.synchronize()
    assert torch.equal(qt2.cpu(), q) and torch.equal(kt2.cpu(), k)
    rp_h = rp.cpu().numpy().astype(np.int64)
    gmask = P.check_csr(rp_h, ci[:int(rp_h[-1])].cpu().numpy(), wl.blocks)
    qbar, kbar, keep, band = P.oracle_select_full(wl, q, k, thr, count_band=True)
    rep = P.compare_masks(gmask, keep, qbar, kbar, wl, thr, band=band)
    P.record_masks(f"partial_raster_{dt}", rep)
    assert P.mask_ok(rep), P.fmt(rep)



# ---------------------------------------------------------------- 4-token key blocks (AB-Attention)

GATHER = [
    # name, heads, d, block grid, thr, reading
    ("d128", 2, 128, (2, 3, 4), 0.8, "A"),
    ("d64_page", 3, 64, (3, 2, 5), 0.9, "page"),
    ("d128_B_odd", 2, 128, (3, 3, 3), 0.9, "B"),
]


@pytest.mark.parametrize("case", GATHER, ids=[c[0] for c in GATHER])
def test_gather_forward_matches_oracle(case):
    """Attention over the oracle's 4-token key blocks, gathered into tiles by the kernel,
    against the oracle's attention over the same blocks, every query block."""
    name, H, d, bg, thr, reading = case
    wl = small_workload("gather_" + name, H, d, bg, "bf16", threshold=thr, seed=91)
    q, k, v, _ = make_inputs(wl, reading)
    qd, kd, vd = P.to_device(q, k, v)
    keep, orp, oci = oracle.select_fine(q, k, H, thr)
    shape = P.shape_for(wl)
    rp = torch.as_tensor(orp.astype(np.int32)).cuda()
    ci = torch.as_tensor(oci).cuda()
    out = torch.full_like(qd, float("nan"))
    lse = torch.full(qd.shape[:3], float("nan"), dtype=torch.float32, device="cuda")
    B.sparse_attn_forward_gather(shape, qd, kd, vd, rp, ci, out=out, lse=lse)
    torch.cuda.synchronize()
    rows = np.arange(H * wl.blocks)
    ref, ref_lse = oracle.attention_rows(q, k, v, orp, oci, rows, key_tokens=4)
    got = out.float().cpu().reshape(-1, 64, d).numpy()
    got_l = lse.cpu().reshape(-1, 64).numpy()
    err = float(np.abs(got - ref).max())
    lerr = float(np.abs(got_l - ref_lse).max())
    print(f"gather {name}: kept {int(keep.sum())} of {keep.size} 4-token blocks, max|err|={err:.3e} lse {lerr:.3e}",
          flush=True)
    assert err <= P.TOL["bf16"] and lerr <= P.LSE_TOL["bf16"]


def test_gather_of_whole_tiles_equals_the_tile_forward():
    """Listing all 16 four-token blocks of each kept tile gathers exactly the tile: the
    output is bit-identical to the tile forward over the tile list.  Junk entries (out of
    range, repeated, descending) are skipped as in the tile forward."""
    wl = small_workload("gather_tiles", 2, 128, (3, 2, 4), "bf16", threshold=0.8, seed=92)
    q, k, v, thr = make_inputs(wl, "A")
    qd, kd, vd = P.to_device(q, k, v)
    qbar, kbar, keep = P.oracle_select_full(wl, q, k, thr)
    orp, oci = oracle.csr_from_mask(keep != 0)
    out_t, lse_t = P.gpu_forward(wl, qd, kd, vd, orp, oci)
    fine = np.repeat(keep != 0, 16, axis=1)
    frp, fci = oracle.csr_from_mask(fine)
    rows = len(frp) - 1
    rp2, ci2 = [0], []
    for r in range(rows):
        seg = fci[frp[r]:frp[r + 1]].tolist()
        ci2 += [-3] + seg[:1] + seg[:1] + seg[1:] + [seg[0], 16 * wl.blocks + 5]
        rp2.append(len(ci2))
    shape = P.shape_for(wl)
    out_g = torch.full_like(qd, float("nan"))
    lse_g = torch.full(qd.shape[:3], float("nan"), dtype=torch.float32, device="cuda")
    B.sparse_attn_forward_gather(shape, qd, kd, vd, torch.as_tensor(np.array(rp2, np.int32)).cuda(),
                                 torch.as_tensor(np.array(ci2, np.int32)).cuda(), out=out_g, lse=lse_g)
    torch.cuda.synchronize()
    assert torch.equal(out_g, out_t) and torch.equal(lse_g, lse_t)


def test_gather_forward_long_lists_and_last_round_pieces():
    """1,024 pairs of query blocks (so the plan cuts the last round of pairs into pieces)
    over random 4-token lists, a few rows far longer than the rest (cut into long-row
    pieces): sampled query blocks of both kinds, and random ones, against the oracle's
    attention over the same list."""
    wl = small_workload("gather_long", 1, 128, (16, 8, 16), "bf16", threshold=0.9, seed=94)
    q, k, v, _ = make_inputs(wl, "A")
    qd, kd, vd = P.to_device(q, k, v)
    nK = 16 * wl.blocks
    rng = np.random.default_rng(95)
    keep = rng.random((wl.blocks, nK)) < 0.03
    long_rows = rng.choice(wl.blocks, 6, replace=False)
    keep[long_rows] = rng.random((6, nK)) < 0.7
    keep[np.arange(wl.blocks), rng.integers(0, nK, wl.blocks)] = True       # no empty row
    orp, oci = oracle.csr_from_mask(keep)
    shape = P.shape_for(wl)
    out, lse = B.sparse_attn_forward_gather(shape, qd, kd, vd, torch.as_tensor(orp.astype(np.int32)).cuda(),
                                            torch.as_tensor(oci).cuda(), want_lse=True)
    torch.cuda.synchronize()
    tail = P.last_round_rows(wl)
    assert tail.size > 0
    rows = np.unique(np.concatenate([tail, long_rows, rng.choice(wl.blocks, 8, replace=False)]))
    ref, ref_lse = oracle.attention_rows(q, k, v, orp, oci, rows, key_tokens=4)
    got = out.float().cpu().reshape(-1, 64, wl.head_dim).numpy()[rows]
    got_l = lse.cpu().reshape(-1, 64).numpy()[rows]
    err = float(np.abs(got - ref).max())
    lerr = float(np.abs(got_l - ref_lse).max())
    print(f"gather long: nnz {len(oci)}, {rows.size} query blocks checked, max|err|={err:.3e} lse {lerr:.3e}",
          flush=True)
    assert err <= P.TOL["bf16"] and lerr <= P.LSE_TOL["bf16"]



@pytest.mark.parametrize("layout", ["same", "interleaved"])
def test_gather_units_of_shared_and_interleaved_rows(layout):
    """Rows whose 4-token lists are identical for every query block (each entry of a pair's
    walk held by both rows, so every position of a unit merges two copies), or split by
    frame parity into even and odd key blocks (the two rows of a frame-neighbour pair then
    alternate entry by entry): every query block against the oracle's attention."""
    wl = small_workload("gather_" + layout, 1, 128, (4, 2, 3), "bf16", seed=96)
    q, k, v, _ = make_inputs(wl, "A")
    qd, kd, vd = P.to_device(q, k, v)
    nB, nK = wl.blocks, 16 * wl.blocks
    rng = np.random.default_rng(97)
    base = rng.random(nK) < 0.6
    keep = np.zeros((nB, nK), dtype=bool)
    per_frame = nB // wl.block_grid[0]
    for i in range(nB):
        if layout == "same":
            keep[i] = base
        else:
            keep[i, (i // per_frame) % 2::2] = True
    orp, oci = oracle.csr_from_mask(keep)
    shape = P.shape_for(wl)
    out, lse = B.sparse_attn_forward_gather(shape, qd, kd, vd, torch.as_tensor(orp.astype(np.int32)).cuda(),
                                            torch.as_tensor(oci).cuda(), want_lse=True)
    torch.cuda.synchronize()
    rows = np.arange(nB)
    ref, ref_lse = oracle.attention_rows(q, k, v, orp, oci, rows, key_tokens=4)
    err = float(np.abs(out.float().cpu().reshape(-1, 64, wl.head_dim).numpy() - ref).max())
    lerr = float(np.abs(lse.cpu().reshape(-1, 64).numpy() - ref_lse).max())
    print(f"gather {layout}: nnz {len(oci)}, max|err|={err:.3e} lse {lerr:.3e}", flush=True)
    assert err <= P.TOL["bf16"] and lerr <= P.LSE_TOL["bf16"]

FINE = [
    # name, heads, d, block grid (nB), thr, reading, per-head threshold range
    ("d128_A_nB24", 2, 128, (2, 3, 4), 0.8, "A", None),            # 1 word a lane
    ("d64_page_nB30", 3, 64, (3, 2, 5), 0.9, "page", None),
    ("d128_B_nB27", 2, 128, (3, 3, 3), 0.9, "B", None),
    ("d128_headthr_nB96", 3, 128, (2, 6, 8), 0.7, "A", (0.5, 0.95)),   # 2 words, ragged rows
    ("d128_page_nB200", 2, 128, (2, 10, 10), 0.85, "page", None),      # 4 words
    ("d64_A_nB480", 1, 64, (5, 8, 12), 0.9, "A", None),                 # 8 words
    ("d128_keepall_nB40", 2, 128, (2, 4, 5), 1.0, "A", None),           # threshold 1: every block
]


def _fine_case(case):
    name, H, d, bg, thr, reading, hr = case
    wl = small_workload("fine_" + name, H, d, bg, "bf16", threshold=thr, head_threshold_range=hr, seed=93)
    q, k, v, th = make_inputs(wl, reading)
    return wl, q, k, v, th


@pytest.mark.parametrize("case", FINE, ids=[c[0] for c in FINE])
def test_fine_selection_matches_oracle(case):
    """4-token key blocks selected per 64-token query block on the GPU against the
    oracle's fine selection: every row, the mask rule of the 64-token selection (R1
    only, no R2-only differences), a valid CSR of ascending 4-token indices."""
    wl, q, k, _, th = _fine_case(case)
    qd, kd = P.to_device(q, k)
    shape = P.shape_for(wl)
    head_thr = None if wl.head_threshold_range is None else [float(x) for x in th]
    rp, ci = B.sparse_attn_select_fine(shape, qd, kd, threshold=float(np.float32(wl.threshold)),
                                       head_thresholds=head_thr)
    torch.cuda.synchronize()
    nK = 16 * wl.blocks
    rp_h = rp.cpu().numpy().astype(np.int64)
    gmask = P.check_csr(rp_h, ci[:int(rp_h[-1])].cpu().numpy(), nK)
    keep, _, _ = oracle.select_fine(q, k, wl.heads, th.astype(np.float64))
    qbar = oracle.pool(q)
    kbar = oracle.pool(k, tpb=4)
    rep = P.compare_masks(gmask, keep.astype(np.uint8), qbar, kbar, wl, th, window=(-1, -1, -1))
    P.record_masks(f"fine_{case[0]}", rep)
    assert P.mask_ok(rep), P.fmt(rep)
    if wl.threshold >= 1.0:
        assert int(rp_h[-1]) == wl.heads * wl.blocks * nK


def test_fine_selection_feeds_the_gather_forward():
    """The GPU's own 4-token list through sparse_attn_forward_gather, against the
    oracle's attention over that same list, every query block."""
    wl, q, k, v, th = _fine_case(("e2e_nB60", 2, 128, (3, 4, 5), 0.85, "page", None))
    qd, kd, vd = P.to_device(q, k, v)
    shape = P.shape_for(wl)
    rp, ci = B.sparse_attn_select_fine(shape, qd, kd, threshold=float(np.float32(wl.threshold)))
    out, lse = B.sparse_attn_forward_gather(shape, qd, kd, vd, rp, ci, want_lse=True)
    torch.cuda.synchronize()
    rp_h = rp.cpu().numpy().astype(np.int64)
    ci_h = ci[:int(rp_h[-1])].cpu().numpy()
    rows = np.arange(wl.heads * wl.blocks)
    ref, ref_lse = oracle.attention_rows(q, k, v, rp_h, ci_h, rows, key_tokens=4)
    err = float(np.abs(out.float().cpu().reshape(-1, 64, wl.head_dim).numpy() - ref).max())
    lerr = float(np.abs(lse.cpu().reshape(-1, 64).numpy() - ref_lse).max())
    print(f"fine e2e: nnz {int(rp_h[-1])} of {rows.size * 16 * wl.blocks}, max|err|={err:.3e} lse {lerr:.3e}",
          flush=True)
    assert err <= P.TOL["bf16"] and lerr <= P.LSE_TOL["bf16"]


def test_fine_selection_uniform_rows_keep_the_lowest_indices():
    """Q = 0: every score is 0, so each row is uniform over its 16 nB key blocks and
    the rule keeps ceil(thr * nK) of them, the lowest indices (all ties)."""
    wl, q, k, _, _ = _fine_case(("uniform_nB64", 1, 128, (1, 8, 8), 0.75, "A", None))
    q = torch.zeros_like(q)
    qd, kd = P.to_device(q, k)
    shape = P.shape_for(wl)
    rp, ci = B.sparse_attn_select_fine(shape, qd, kd, threshold=0.75)
    torch.cuda.synchronize()
    nK = 16 * wl.blocks
    want = int(np.ceil(0.75 * nK))
    rp_h = rp.cpu().numpy().astype(np.int64)
    assert np.all(np.diff(rp_h) == want)
    ci_h = ci[:int(rp_h[-1])].cpu().numpy().reshape(wl.blocks, want)
    assert np.all(ci_h == np.arange(want)[None, :])
