"""Helpers for the GPU parity tests: run the HIP path through the C-ABI binding
and compare it with the CPU oracle.

Mask rule (selection).  Where GPU and oracle disagree on block j of a row,
with p, E the oracle's probabilities and exclusive CDF mass and c the
oracle's crossing block (the last block it keeps in CDF order):
  R1  excused if |E(j) - thr| <= 1e-4;
  R2  excused (when R1 does not excuse it) if |p_j - p_c| <= 1e-5 * p_c: a rank
      swap of near-equal blocks at the cut, which moves E(j) by a whole p_c;
window blocks are never excused.  On every row that disagrees, the GPU's CDF
set (the oracle's CDF set with the differing blocks toggled: those are never
window blocks) must hold mass >= thr - 1e-4 and stay minimal (mass minus its
smallest block < thr + 1e-4).  The counts (R1 only,
R2 only, blocks inside the R1 band over all rows, the largest mass deviation)
are returned, and written as JSON to $SPARSE_ATTN_PARITY_DIR when it is set.
"""
from __future__ import annotations

import json
import math
import os
from dataclasses import dataclass

import numpy as np
import torch

import oracle
from block_sparse_attention_row_amd import binding as B
from block_sparse_attention_row_amd.synth import Workload

R1_BAND = 1e-4
R2_REL = 1e-5
TOL = {"bf16": 2e-2, "f32": 1e-4}
# The bf16 path normalises with the sum of the same bf16-rounded weights that enter
# P V, so its log-sum-exp carries up to the bf16 unit roundoff 2^-8 ~ 3.9e-3 of
# relative error in the normaliser; fp32 keeps fp32 weights.
LSE_TOL = {"bf16": 5e-3, "f32": 1e-4}


def forward_tols(dtype: str, reading: str):
    """(output, LSE) bounds of a forward against the oracle.  Reading B gives logits near
    200: a 128-term fp32 dot product of that size carries about sqrt(d) * ulp(2048) / 2
    ~ 7e-4 of rounding (6e-5 after the 1/sqrt(d) scale), which moves the softmax weights
    by that relative amount; 1e-3 covers it with margin.  The 1e-4 fp32 bound is for
    logits of O(1) (reading A and the specified fp32 workload)."""
    if dtype == "f32" and reading != "A":
        return 1e-3, 1e-3
    return TOL[dtype], LSE_TOL[dtype]
# Backward (bf16): max |GPU - oracle| over max |oracle|, per gradient.  The kernels
# round P (for dV) and dS (for dQ, dK) to bf16 before the MFMA products.  bf16 keeps
# 8 significand bits, so its unit roundoff (half an ulp of 1) is u = 2^-8 = 3.9e-3
# per rounded term.  dV = sum_n P dO has nonnegative weights, so the roundings of P
# (relative, at most u each, of random sign) average out and its error stays below
# u times max |dV|: BWD_TOL_DV = 1.28u = 5e-3.  Each row of dS sums to zero
# (sum_m P (dP - D) = D - D), so dQ = scale sum_m dS k_m cancels the keys' common part
# and dK likewise; the rounding error scales with sum |dS| |k| instead, which was 5-9
# times max |dQ| on the test inputs (checked by an fp64 emulation of the roundings,
# which gives the GPU's errors to within a few percent).  When the oracle recomputes O
# exactly while the kernels read the bf16 forward output, D = dO . O carries a further
# |dO| |O| u, passed into dS the same way.  BWD_TOL_DQK = 5.1u = 2e-2 covers both.
BWD_TOL_DV = 5e-3
BWD_TOL_DQK = 2e-2
# Backward (fp32): P and dS stay fp32 (u = 2^-24 per rounding, v_exp_f32 within a few
# ulps), so the errors are those of fp32 sums over the kept keys, times the same
# cancellation factor of up to ~9 in dQ and dK, and D taken from the fp32 forward
# output (1e-4 absolute, TOL["f32"]) when the oracle recomputes O in fp64.  One bound
# for all three gradients: the fp32 forward's, 1e-4 of max |ref|.
BWD_TOL_F32 = 1e-4


def to_device(*ts):
    return [t.to("cuda") for t in ts]


def shape_for(wl: Workload) -> B.Shape:
    return B.make_shape(wl.batch, wl.heads, wl.head_dim, wl.grid, wl.dtype, 0.0, wl.tile)


def check_csr(row_ptr: np.ndarray, col_idx: np.ndarray, nB: int):
    """Structural validity of a CSR block list; returns the dense mask."""
    rows = len(row_ptr) - 1
    assert row_ptr[0] == 0
    assert np.all(np.diff(row_ptr) >= 0)
    nnz = int(row_ptr[-1])
    cols = col_idx[:nnz]
    assert np.all((cols >= 0) & (cols < nB))
    mask = np.zeros((rows, nB), dtype=bool)
    r = np.repeat(np.arange(rows), np.diff(row_ptr))
    # strictly ascending within each row
    same = r[1:] == r[:-1]
    assert np.all(cols[1:][same] > cols[:-1][same])
    mask[r, cols] = True
    return mask


def gpu_select(wl: Workload, q, k, thr, window=None, bufs=None):
    shape = shape_for(wl)
    win = wl.window if window is None else window
    head_thr = None if wl.head_threshold_range is None else [float(x) for x in thr]
    bufs = bufs or B.alloc_buffers(shape, q.device)
    rp, ci = B.sparse_attn_select(shape, q, k, threshold=float(np.float32(wl.threshold)),
                                  head_thresholds=head_thr, window=win, buffers=bufs)
    assert B.sparse_attn_select_check(shape, bufs.workspace) == B.SPARSE_ATTN_OK
    torch.cuda.synchronize()
    rp_h = rp.cpu().numpy().astype(np.int64)
    nnz = int(rp_h[-1])
    ci_h = ci[:nnz].cpu().numpy()
    return rp_h, ci_h


@dataclass
class MaskReport:
    rows: int
    diff_rows: int
    diff_blocks: int
    r1: int                  # differing blocks excused by R1
    r2: int                  # differing blocks excused by R2 only
    unexcused: int
    window_missing: int
    invariant_fail: int
    band: int = -1           # blocks inside the R1 band over all rows (-1: not counted)
    mass_dev: float = 0.0    # largest |GPU CDF-set mass - oracle CDF-set mass| on differing rows

    def as_dict(self):
        return dict(self.__dict__)


def compare_masks(gpu_mask: np.ndarray, keep: np.ndarray, qbar, kbar, wl: Workload, thr: np.ndarray,
                  window=None, band: int = -1) -> MaskReport:
    """gpu_mask, keep: [rows, nK]; keep is the oracle's (bit0 CDF, bit1 window).  kbar
    holds the key blocks of the rows: nK = nB (64-token blocks) or 16 nB (4-token
    blocks, with the window off)."""
    win = wl.window if window is None else window
    nB = wl.blocks      # query blocks per head: row r belongs to head (r // nB) % H
    oracle_mask = keep != 0
    diff = np.nonzero((gpu_mask != oracle_mask).any(axis=1))[0]
    r1 = r2 = unexc = wmiss = inv = nblk = 0
    mass_dev = 0.0
    if len(diff):
        kk, p, E = oracle.select_rows(qbar, kbar, wl.heads, wl.block_grid, thr.astype(np.float64), win,
                                      rows=diff, stats=True)
        for n, r in enumerate(diff):
            t = float(thr[(r // nB) % wl.heads])
            cdf = (kk[n] & 1) != 0
            if t >= 1.0:
                pc = None
            else:
                c = int(np.argmax(np.where(cdf, E[n], -1.0)))
                pc = p[n, c]
            dj = np.nonzero(gpu_mask[r] != oracle_mask[r])[0]
            for j in dj:
                nblk += 1
                if kk[n, j] & 2:
                    wmiss += 1
                    continue
                if abs(E[n, j] - t) <= R1_BAND:
                    r1 += 1
                elif pc is not None and abs(p[n, j] - pc) <= R2_REL * pc:
                    r2 += 1
                else:
                    unexc += 1
            if t < 1.0:
                # the GPU's CDF set: the oracle's with the differing (non-window) blocks toggled
                g = cdf.copy()
                g[dj] = ~g[dj]
                kp = p[n][g]
                m = float(kp.sum()) if kp.size else 0.0
                if not (kp.size and m >= t - R1_BAND and m - kp.min() < t + R1_BAND):
                    inv += 1
                mass_dev = max(mass_dev, abs(m - float(p[n][cdf].sum())))
    return MaskReport(gpu_mask.shape[0], len(diff), nblk, r1, r2, unexc, wmiss, inv, band, mass_dev)


def mask_ok(rep: MaskReport) -> bool:
    """The spec rule: every difference within R1's band of the threshold (R2-only
    differences are counted but not accepted), no window block missing, and the GPU's
    set valid."""
    return rep.unexcused == 0 and rep.r2 == 0 and rep.window_missing == 0 and rep.invariant_fail == 0


def record_masks(label: str, rep: MaskReport, **extra):
    """Print the mask report and, with $SPARSE_ATTN_PARITY_DIR set, keep it as JSON."""
    print(f"[masks] {label}: {fmt(rep)}", flush=True)
    d = os.environ.get("SPARSE_ATTN_PARITY_DIR")
    if d:
        os.makedirs(d, exist_ok=True)
        rec = dict(label=label, **rep.as_dict(), **extra)
        with open(os.path.join(d, f"masks_{label}.json"), "w") as f:
            json.dump(rec, f, indent=1)


def valid_of(wl: Workload):
    """The tile-major slots that are grid tokens, or None when every tile is whole."""
    return oracle.token_valid(wl.grid, wl.tile) if wl.partial else None


def oracle_select_full(wl: Workload, q, k, thr, window=None, count_band: bool = False, chunk: int = 2048):
    """The oracle's selection for every row: (qbar, kbar, keep) and, with count_band,
    also the number of blocks whose exclusive mass lies within R1_BAND of the
    threshold (the blocks R1 could excuse), counted chunk by chunk."""
    win = wl.window if window is None else window
    qbar = oracle.pool(q, valid=valid_of(wl))
    kbar = oracle.pool(k, valid=valid_of(wl))
    th = thr.astype(np.float64)
    if not count_band:
        return qbar, kbar, oracle.select_rows(qbar, kbar, wl.heads, wl.block_grid, th, win)
    rows = wl.batch * wl.heads * wl.blocks
    keep = np.empty((rows, wl.blocks), dtype=np.uint8)
    band = 0
    for r0 in range(0, rows, chunk):
        rr = np.arange(r0, min(rows, r0 + chunk))
        kk, _, E = oracle.select_rows(qbar, kbar, wl.heads, wl.block_grid, th, win, rows=rr, stats=True)
        keep[rr] = kk
        t = th[(rr // wl.blocks) % wl.heads][:, None]
        band += int(((np.abs(E - t) <= R1_BAND) & (t < 1.0)).sum())
    return qbar, kbar, keep, band


def gpu_forward(wl: Workload, q, k, v, row_ptr, col_idx, want_lse=True):
    shape = shape_for(wl)
    rp = torch.as_tensor(np.asarray(row_ptr, dtype=np.int32)).cuda()
    ci = torch.as_tensor(np.asarray(col_idx, dtype=np.int32)).cuda()
    if ci.numel() == 0:
        ci = torch.zeros(1, dtype=torch.int32, device="cuda")[:0]
    out = torch.full_like(q, float("nan"))
    lse = torch.full(q.shape[:3], float("nan"), dtype=torch.float32, device=q.device)
    B.sparse_attn_forward(shape, q, k, v, rp, ci, out=out, lse=lse)
    torch.cuda.synchronize()
    return out, lse


def compare_rows(wl: Workload, out, lse, q, k, v, row_ptr, col_idx, rows, bias=None):
    """Max |GPU - oracle| of output and LSE over the listed query-block rows (padding
    slots of partial tiles included: both sides must give O = 0, LSE = -inf there)."""
    ref, ref_lse = oracle.attention_rows(q, k, v, row_ptr, col_idx, rows, bias=bias, valid=valid_of(wl))
    nB = wl.blocks
    o = out.float().cpu().reshape(-1, nB, 64, wl.head_dim)
    l = lse.cpu().reshape(-1, nB, 64)
    rows = np.asarray(rows)
    got = o[rows // nB, rows % nB].numpy().astype(np.float64)
    got_l = l[rows // nB, rows % nB].numpy().astype(np.float64)
    assert np.isfinite(got).all(), "non-finite output"
    err = float(np.abs(got - ref).max()) if got.size else 0.0
    fin = np.isfinite(ref_lse)
    assert np.array_equal(np.isneginf(got_l), ~fin)
    lerr = float(np.abs(got_l[fin] - ref_lse[fin]).max()) if fin.any() else 0.0
    return err, lerr


def gpu_forward_biased(wl: Workload, q, k, v, row_ptr, col_idx, bias):
    shape = shape_for(wl)
    rp = torch.as_tensor(np.asarray(row_ptr, dtype=np.int32)).cuda()
    ci = torch.as_tensor(np.asarray(col_idx, dtype=np.int32)).cuda()
    cb = torch.as_tensor(np.asarray(bias, dtype=np.float32)).cuda()
    out = torch.full_like(q, float("nan"))
    lse = torch.full(q.shape[:3], float("nan"), dtype=torch.float32, device=q.device)
    B.sparse_attn_forward_biased(shape, q, k, v, rp, ci, cb, out=out, lse=lse)
    torch.cuda.synchronize()
    return out, lse


# Sampling with inclusion probabilities: the kernels form pi from fp32 exponentials of
# split-bf16 pooled scores (relative error near 2^-16 of the score, up to ~1e-4 of pi
# after exponentiation and the normalising constant).  A kept-set difference is
# excused when the block's uniform lies within SIP_BAND * pi of the oracle's pi; the
# offsets of blocks kept by both agree to SIP_BIAS_TOL (|d ln pi| ~ |d pi / pi|).
SIP_BAND = 1e-3
SIP_BIAS_TOL = 2e-3


def compare_sip(rp_g: np.ndarray, ci_g: np.ndarray, cb_g: np.ndarray, keep, pi, u, nB: int):
    """(differing blocks, unexcused differences, max offset error on common blocks)."""
    gmask = check_csr(rp_g, ci_g, nB)
    diff = gmask != keep
    unexcused = int((diff & ~(np.abs(u - pi) <= SIP_BAND * pi)).sum())
    rows = np.repeat(np.arange(len(rp_g) - 1), np.diff(rp_g))
    both = keep[rows, ci_g[:len(rows)]]
    ref = -np.log(pi[rows, ci_g[:len(rows)]])
    berr = float(np.abs(cb_g[:len(rows)][both] - ref[both]).max()) if both.any() else 0.0
    return int(diff.sum()), unexcused, berr


# Clustering selector: the GPU forms centroids as fp32 means and p~ with fp32
# exponentials of fp32 dot products (key means as hi + lo bf16), so p~ carries
# about 1e-5 relative error against the fp64 oracle.  The squared distances of the
# assignment carry ~1e-6 relative error (fp32 sums of 128 squares, centroids that
# are fp32 means); a pair whose k-means came within IBCS_GAP (relative) of an
# assignment tie in the oracle may cluster differently: its rows are checked for
# validity only.  Elsewhere a kept-set
# difference is excused at the CDF boundary: the mass before the block within
# IBCS_BAND_E of the threshold, or its p~ within IBCS_BAND_P (relative) of the
# crossing block's.
IBCS_GAP = 1e-5
IBCS_BAND_E = 1e-4
IBCS_BAND_P = 1e-4


def compare_cdf_rows(gmask: np.ndarray, keep: np.ndarray, p: np.ndarray, thr_rows: np.ndarray,
                     skip: np.ndarray):
    """(differing blocks, excused, unexcused) over the rows not in `skip`; window-free."""
    ndiff = nexc = nunx = 0
    for r in np.nonzero((gmask != keep).any(axis=1) & ~skip)[0]:
        order = np.argsort(-p[r], kind="stable")
        before = np.empty(p.shape[1])
        before[order] = np.concatenate([[0.0], np.cumsum(p[r][order])[:-1]])
        kept = order[keep[r][order]]
        pc = p[r][kept[-1]] if len(kept) else 0.0
        for j in np.nonzero(gmask[r] != keep[r])[0]:
            ndiff += 1
            if abs(before[j] - thr_rows[r]) <= IBCS_BAND_E or abs(p[r][j] - pc) <= IBCS_BAND_P * pc:
                nexc += 1
            else:
                nunx += 1
    return ndiff, nexc, nunx


def sample_rows(wl: Workload, thr: np.ndarray, n_heads=2, n_blocks=32, seed=1):
    rng = np.random.default_rng(seed)
    if wl.head_threshold_range is not None:
        heads = [int(np.argmin(thr)), int(np.argmax(thr))]
    else:
        heads = sorted(rng.choice(wl.heads, size=min(n_heads, wl.heads), replace=False).tolist())
    rows = []
    for h in heads:
        blocks = np.sort(rng.choice(wl.blocks, size=min(n_blocks, wl.blocks), replace=False))
        rows.extend((h * wl.blocks + blocks).tolist())        # batch 0
    return np.array(rows, dtype=np.int64)


# The bf16 forward's launch order (host-side mirror, for choosing test rows): whole
# pairs are dispatched in the order of xcd_chunk_remap<256>, and with at least two
# rounds of resident pairs (512) the last 384 of them are cut into pieces that run
# at the end of the launch.
def _xcd_remap(bid, n, x8=8):
    x, k = bid % x8, bid // x8
    per, rem = n // x8, n % x8
    return x * per + min(x, rem) + k


def _xcd_chunk_remap(bid, n, c=256, x8=8):
    full = n // (x8 * c) * (x8 * c)
    if bid >= full:
        return full + _xcd_remap(bid - full, n - full)
    x, k = bid % x8, bid // x8
    return (k // c) * (x8 * c) + x * c + k % c


def pair_blocks(p, s, nb):
    """Blocks of query-block pair p of a head in the forward: frame-neighbours (stride
    s = blocks per frame), an odd last frame side by side; -1 for no second block."""
    nt = nb // s
    full = (nt // 2) * s
    if p < full:
        u, r = divmod(p, s)
        return 2 * u * s + r, 2 * u * s + r + s
    s2 = p - full
    a = (nt - 1) * s + 2 * s2
    return a, (a + 1 if 2 * s2 + 1 < s else -1)


def pair_stride(wl: Workload):
    nt, ny, nx = wl.block_grid
    return ny * nx if nt >= 2 else 1


def last_round_rows(wl: Workload, n_pairs_picked=6):
    """Query blocks (global rows, batch 0 first) of some pairs the forward cuts into
    last-round pieces; empty when the workload has fewer than two rounds of pairs."""
    pph = (wl.blocks + 1) // 2
    n = wl.batch * wl.heads * pph
    if n < 2 * 512:
        return np.zeros(0, dtype=np.int64)
    picks = np.linspace(n - 384, n - 1, n_pairs_picked).round().astype(np.int64)
    rows = []
    for b in picks:
        p = _xcd_chunk_remap(int(b), n)
        bh, i = divmod(p, pph)
        ba, bb = pair_blocks(i, pair_stride(wl), wl.blocks)
        rows.append(bh * wl.blocks + ba)
        if bb >= 0:
            rows.append(bh * wl.blocks + bb)
    return np.array(rows, dtype=np.int64)


def flops_kept(nnz: int, d: int) -> float:
    return 4.0 * 64 * 64 * d * nnz


def fmt(rep: MaskReport) -> str:
    return (f"rows={rep.rows} diff_rows={rep.diff_rows} diff_blocks={rep.diff_blocks} R1={rep.r1} R2only={rep.r2} "
            f"unexcused={rep.unexcused} window_missing={rep.window_missing} invariant_fail={rep.invariant_fail} "
            f"band={rep.band} mass_dev={rep.mass_dev:.2e}")


def scale_of(d: int) -> float:
    return 1.0 / math.sqrt(d)


def backward_sampled(wl, shape, qd, kd, vd, lse, q32, k32, v32, orp, oci, sample, log=print):
    """The backward at full size over the oracle's whole block list, with the upstream
    gradient nonzero only on a few sampled query-block rows: the gradients are linear
    in it and a row with dO = 0 adds exact zeros, so every gradient entry comes from
    those rows, which the oracle computes under the block list cut down to them.  Both
    sides take D = dO . O from the oracle's forward output of those rows, in bf16."""
    nB, d = wl.blocks, wl.head_dim
    rows_s = np.sort(sample[:: max(1, len(sample) // 6)][:6])
    o_ref, _ = oracle.attention_rows(q32, k32, v32, orp, oci, rows_s)
    o_in = torch.zeros(q32.shape, dtype=torch.bfloat16).reshape(-1, 64, d)
    dout = torch.zeros_like(o_in)
    gen = torch.Generator().manual_seed(12)
    o_in[rows_s] = torch.as_tensor(o_ref).to(torch.bfloat16)
    dout[rows_s] = torch.randn((len(rows_s), 64, d), generator=gen).to(torch.bfloat16)
    o_in, dout = o_in.reshape(q32.shape), dout.reshape(q32.shape)
    rpd = torch.as_tensor(orp.astype(np.int32)).cuda()
    cid = torch.as_tensor(oci).cuda()
    dq, dk, dv = B.sparse_attn_backward(shape, qd, kd, vd, o_in.cuda(), lse, dout.cuda(), rpd, cid)
    torch.cuda.synchronize()
    log(f"backward done on the GPU; oracle over rows {rows_s.tolist()}")
    keep = np.zeros(len(orp) - 1, dtype=bool)
    keep[rows_s] = True
    lens = np.diff(orp)
    rp_s = np.concatenate([[0], np.cumsum(np.where(keep, lens, 0))])
    ci_s = np.concatenate([oci[orp[r]:orp[r + 1]] for r in rows_s])
    rq, rk, rv = oracle.attention_backward(q32, k32, v32, dout.float().numpy(), rp_s, ci_s, out=o_in.float().numpy(),
                                           valid=valid_of(wl))
    errs = []
    for name, got, ref in (("dq", dq, rq), ("dk", dk, rk), ("dv", dv, rv)):
        g = got.float().cpu().numpy()
        assert np.all(g[ref == 0] == 0), name          # rows with dO = 0 add exact zeros
        errs.append(float(np.abs(g - ref).max() / np.abs(ref).max()))
    log(f"backward, {len(rows_s)} sampled rows: rel err dq {errs[0]:.3e} dk {errs[1]:.3e} dv {errs[2]:.3e}")
    assert max(errs[:2]) <= BWD_TOL_DQK and errs[2] <= BWD_TOL_DV


# ------------------------------------------------------------- mask record summary
_SUMMARY_HEAD = """# Mask parity records (GPU selection against the fp64 oracle)

Every row of every listed case: the GPU's block list against the oracle's.  `diff` = blocks on which the two
differ; `R1` = differences excused because the oracle's exclusive mass E(j) lies within 1e-4 of the threshold;
`R2` = differences only a near-tie rule would excuse (|p_j - p_c| <= 1e-5 p_c) -- counted, never accepted;
`unexcused` must be 0; `window missing` = window blocks the GPU left out (must be 0); `invariant` = rows
whose GPU set fails kept mass >= thr - 1e-4 or minimality (must be 0); `band` = blocks within R1's band over
all rows (where R1 could excuse a difference), counted on the full-size cases; `nnz` = kept tiles, GPU / oracle.

Made from the JSON records of a GPU suite run (from the repository root on an MI355X, after building in-tree):

```
SPARSE_ATTN_PARITY_DIR=<out> python -u -m pytest tests/ -x -v -m gpu --timeout 900 --timeout-method thread
python -m tests.parity --summary <out> > profiles/parity_masks.md
```

Full-size cases are the five workloads (and the B and page-like readings of two of them, and `partial_480p`: a
20 x 30 x 45 token grid, 480 blocks whose last tile row and column are partial); `fine_*` is the
selection of 4-token key blocks (16 nB key blocks a row).
"""


def summarize(directory: str) -> str:
    """The markdown table of every masks_*.json record in `directory`."""
    import glob
    recs = []
    for path in sorted(glob.glob(os.path.join(directory, "masks_*.json"))):
        with open(path) as f:
            recs.append(json.load(f))
    lines = [_SUMMARY_HEAD, "| case | rows | diff rows | diff | R1 | R2 | unexcused | window missing | invariant | band | nnz |",
             "|---|---|---|---|---|---|---|---|---|---|---|"]
    for r in sorted(recs, key=lambda r: r["label"]):
        band = r.get("band", -1)
        nnz = f"{r['nnz']} / {r['oracle_nnz']}" if "nnz" in r and "oracle_nnz" in r else "-"
        lines.append(f"| {r['label']} | {r['rows']} | {r['diff_rows']} | {r['diff_blocks']} | {r['r1']} | {r['r2']} | "
                     f"{r['unexcused']} | {r['window_missing']} | {r['invariant_fail']} | "
                     f"{band if band >= 0 else '-'} | {nnz} |")
    tot = {k: sum(r[k] for r in recs) for k in ("diff_blocks", "r1", "r2", "unexcused", "window_missing", "invariant_fail")}
    lines.append("")
    lines.append(f"{len(recs)} cases; over all of them: {tot['diff_blocks']} differing blocks, {tot['r1']} excused by R1, "
                 f"{tot['r2']} R2-only, {tot['unexcused']} unexcused, {tot['window_missing']} window blocks missing, "
                 f"{tot['invariant_fail']} invariant failures.")
    return "\n".join(lines) + "\n"


if __name__ == "__main__":
    import argparse
    ap = argparse.ArgumentParser(description="summaries of the GPU parity records")
    ap.add_argument("--summary", required=True, help="directory of masks_*.json records")
    print(summarize(ap.parse_args().summary), end="")
