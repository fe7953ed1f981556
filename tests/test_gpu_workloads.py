"""GPU parity at the full sizes of the four video-DiT workloads (plus the tiny
fp32 one in test_gpu_parity.py), in the launch configuration bench.py times.

Selection: every row of every head is compared with the oracle under the
mask rule in parity.py, under reading A on all four grids and under reading B
and the page-like variant on the 480p and long-video grids.  Attention: every
query block of the 480p workload under the oracle's block list; on the larger
grids sampled query blocks (2 heads x 32 blocks, drawn with rng(1); for the
jittered-threshold workload the heads with the lowest and highest threshold,
and 12 blocks of pairs the forward cuts into last-round pieces) under the
oracle's block list, and the same rows under the GPU's own block list where
the two masks agree.  Backward (bf16):
dQ, dK, dV over the whole block list with the upstream gradient on six of the
sampled rows (see _backward_sampled).
"""
import time

import numpy as np
import pytest
import torch

import oracle
from block_sparse_attention_row_amd import binding as B
from block_sparse_attention_row_amd.synth import WORKLOADS, make_inputs

from . import parity as P

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

BIG = ["wan13b_480p", "wan14b_720p", "hunyuan_720p", "long_video"]


def _log(msg):
    print(f"[{time.strftime('%H:%M:%S')}] {msg}", flush=True)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", BIG)
def test_full_size_workload(name):
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a ROCm GPU")
    wl = WORKLOADS[name]
    _log(f"[case] {name}: drawing inputs ({wl.description})")
    q, k, v, thr = make_inputs(wl, "A")
    qd, kd, vd = P.to_device(q, k, v)
    shape = P.shape_for(wl)
    bufs = B.alloc_buffers(shape)

    # the GPU path as bench.py runs it: select, then forward on the same buffers
    head_thr = None if wl.head_threshold_range is None else [float(x) for x in thr]
    rp, ci = B.sparse_attn_select(shape, qd, kd, threshold=float(np.float32(wl.threshold)),
                                  head_thresholds=head_thr, window=wl.window, buffers=bufs)
    out_g = torch.empty_like(qd)
    lse_g = torch.empty(qd.shape[:3], dtype=torch.float32, device="cuda")
    B.sparse_attn_forward(shape, qd, kd, vd, rp, ci, out=out_g, lse=lse_g, workspace=bufs.workspace)
    torch.cuda.synchronize()
    rp_h = rp.cpu().numpy().astype(np.int64)
    ci_h = ci[:int(rp_h[-1])].cpu().numpy()
    gmask = P.check_csr(rp_h, ci_h, wl.blocks)
    rows = wl.batch * wl.heads * wl.blocks
    _log(f"GPU done: nnz={int(rp_h[-1])} kept={rp_h[-1] / (rows * wl.blocks):.4f}")

    # exact fp32 copies for the oracle, made once
    q32, k32, v32 = (t.float().numpy() for t in (q, k, v))
    qbar, kbar, keep, band = P.oracle_select_full(wl, q32, k32, thr, count_band=True)
    rep = P.compare_masks(gmask, keep, qbar, kbar, wl, thr, band=band)
    P.record_masks(f"{name}_A", rep, nnz=int(rp_h[-1]), oracle_nnz=int((keep != 0).sum()))
    assert P.mask_ok(rep), P.fmt(rep)

    # the 480p workload: every query block under the oracle's list; the larger ones:
    # sampled blocks, plus blocks of pairs that the forward cuts into last-round pieces
    orp, oci = oracle.csr_from_mask(keep != 0)
    sample = np.unique(np.concatenate([P.sample_rows(wl, thr), P.last_round_rows(wl)]))
    checked = np.arange(rows) if name == "wan13b_480p" else sample
    out_o, lse_o = P.gpu_forward(wl, qd, kd, vd, orp, oci)
    t0 = time.time()
    err, lerr = P.compare_rows(wl, out_o, lse_o, q32, k32, v32, orp, oci, checked)
    _log(f"forward (oracle CSR), {len(checked)} of {rows} query blocks: max|err|={err:.3e} "
         f"lse max|err|={lerr:.3e} (oracle {time.time() - t0:.1f} s)")
    assert err <= P.TOL[wl.dtype] and lerr <= P.LSE_TOL[wl.dtype]

    agree = sample[~(gmask[sample] != (keep[sample] != 0)).any(axis=1)]
    err2, lerr2 = P.compare_rows(wl, out_g, lse_g, q32, k32, v32, orp, oci, agree)
    _log(f"forward (GPU CSR), {len(agree)} sampled blocks with equal masks: max|err|={err2:.3e} "
         f"lse max|err|={lerr2:.3e}")
    assert err2 <= P.TOL[wl.dtype] and lerr2 <= P.LSE_TOL[wl.dtype]
    if wl.dtype == "bf16":
        P.backward_sampled(wl, shape, qd, kd, vd, lse_o, q32, k32, v32, orp, oci, sample, log=_log)


@pytest.mark.timeout(600)
def test_full_size_partial_tiles():
    """A grid of the 480p workload's size that is not a whole number of tiles
    (20 x 30 x 45 tokens in 1 x 8 x 8 tiles: 480 blocks, the last row and column of
    tiles partial), junk in every padding slot: every mask row against the oracle,
    sampled query blocks of the forward under the oracle's list (padding slots O = 0),
    and the sampled backward (padding slots zero gradients)."""
    from block_sparse_attention_row_amd.synth import Workload
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a ROCm GPU")
    wl = Workload("partial_480p", 1, 12, 128, (20, 30, 45), "bf16", 2.0, 0.9, seed=23)
    assert wl.partial and wl.blocks == 480
    _log(f"[case] {wl.name}: drawing inputs (grid {wl.grid}, {wl.blocks} blocks)")
    q, k, v, thr = make_inputs(wl, "A")
    valid = torch.as_tensor(P.valid_of(wl))
    for t in (q, k, v):
        t[..., ~valid, :] = 7.0
    qd, kd, vd = P.to_device(q, k, v)
    shape = P.shape_for(wl)
    rp_h, ci_h = P.gpu_select(wl, qd, kd, thr)
    gmask = P.check_csr(rp_h, ci_h, wl.blocks)
    rows = wl.batch * wl.heads * wl.blocks
    _log(f"GPU selection done: nnz={int(rp_h[-1])} kept={rp_h[-1] / (rows * wl.blocks):.4f}")
    q32, k32, v32 = (t.float().numpy() for t in (q, k, v))
    qbar, kbar, keep, band = P.oracle_select_full(wl, q32, k32, thr, count_band=True)
    rep = P.compare_masks(gmask, keep, qbar, kbar, wl, thr, band=band)
    P.record_masks(wl.name, rep, nnz=int(rp_h[-1]), oracle_nnz=int((keep != 0).sum()))
    assert P.mask_ok(rep), P.fmt(rep)
    orp, oci = oracle.csr_from_mask(keep != 0)
    sample = np.unique(np.concatenate([P.sample_rows(wl, thr), P.last_round_rows(wl)]))
    out_o, lse_o = P.gpu_forward(wl, qd, kd, vd, orp, oci)
    err, lerr = P.compare_rows(wl, out_o, lse_o, q32, k32, v32, orp, oci, sample)
    _log(f"forward (oracle CSR), {len(sample)} sampled blocks: max|err|={err:.3e} lse max|err|={lerr:.3e}")
    assert err <= P.TOL[wl.dtype] and lerr <= P.LSE_TOL[wl.dtype]
    assert torch.all(out_o.cpu()[..., ~valid, :] == 0)
    P.backward_sampled(wl, shape, qd, kd, vd, lse_o, q32, k32, v32, orp, oci, sample, log=_log)


OTHER_READINGS = [(n, r) for n in ("wan13b_480p", "long_video") for r in ("B", "page")]


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name,reading", OTHER_READINGS, ids=[f"{n}-{r}" for n, r in OTHER_READINGS])
def test_full_size_other_readings(name, reading):
    """The two other generator readings at full size: reading B (1-4 kept blocks a row)
    and the page-like variant (about 10% kept, rows from one to hundreds of tiles, the
    sparsity the pages report).  Every mask row against the oracle, then sampled query
    blocks of the forward under the oracle's list."""
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a ROCm GPU")
    wl = WORKLOADS[name]
    _log(f"[case] {name} reading {reading}: drawing inputs")
    q, k, v, thr = make_inputs(wl, reading)
    qd, kd, vd = P.to_device(q, k, v)
    shape = P.shape_for(wl)
    rp_h, ci_h = P.gpu_select(wl, qd, kd, thr)
    gmask = P.check_csr(rp_h, ci_h, wl.blocks)
    rows = wl.batch * wl.heads * wl.blocks
    _log(f"GPU selection done: nnz={int(rp_h[-1])} kept={rp_h[-1] / (rows * wl.blocks):.4f}")
    q32, k32, v32 = (t.float().numpy() for t in (q, k, v))
    qbar, kbar, keep, band = P.oracle_select_full(wl, q32, k32, thr, count_band=True)
    rep = P.compare_masks(gmask, keep, qbar, kbar, wl, thr, band=band)
    P.record_masks(f"{name}_{reading}", rep, nnz=int(rp_h[-1]), oracle_nnz=int((keep != 0).sum()))
    assert P.mask_ok(rep), P.fmt(rep)
    orp, oci = oracle.csr_from_mask(keep != 0)
    sample = np.unique(np.concatenate([P.sample_rows(wl, thr), P.last_round_rows(wl)]))
    out_o, lse_o = P.gpu_forward(wl, qd, kd, vd, orp, oci)
    err, lerr = P.compare_rows(wl, out_o, lse_o, q32, k32, v32, orp, oci, sample)
    _log(f"forward (oracle CSR), {len(sample)} sampled blocks: max|err|={err:.3e} lse max|err|={lerr:.3e}")
    assert err <= P.TOL[wl.dtype] and lerr <= P.LSE_TOL[wl.dtype]


@pytest.mark.timeout(600)
def test_sip_full_size_480p():
    """Sampling with inclusion probabilities at full size (budget of 10% of the key
    blocks, as sparse as the AB-Attention page's runs): every row's sampled set and
    offsets against the oracle, and the offset forward on sampled rows under the
    oracle's list."""
    from oracle import sip
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a ROCm GPU")
    wl = WORKLOADS["wan13b_480p"]
    budget = 0.1 * wl.blocks
    _log(f"[case] SIP {wl.name} budget {budget}")
    q, k, v, thr = make_inputs(wl, "A")
    qd, kd, vd = P.to_device(q, k, v)
    shape = P.shape_for(wl)
    rp, ci, cb = B.sparse_attn_select_sip(shape, qd, kd, budget, seed=2026)
    torch.cuda.synchronize()
    rp_h = rp.cpu().numpy().astype(np.int64)
    nnz = int(rp_h[-1])
    q32, k32, v32 = (t.float().numpy() for t in (q, k, v))
    keep, orp, oci, obias, pi, u = sip.select_sip(q32, k32, wl.heads, budget, seed=2026)
    ndiff, unexcused, berr = P.compare_sip(rp_h, ci[:nnz].cpu().numpy(), cb[:nnz].cpu().numpy(), keep, pi, u,
                                           wl.blocks)
    _log(f"SIP: kept {nnz} (oracle {int(keep.sum())}, expected {budget * wl.heads * wl.blocks:.0f}), "
         f"differing {ndiff}, unexcused {unexcused}, max offset err {berr:.2e}")
    assert unexcused == 0 and berr <= P.SIP_BIAS_TOL
    sample = P.sample_rows(wl, thr)
    out, lse = P.gpu_forward_biased(wl, qd, kd, vd, orp, oci, obias.astype(np.float32))
    err, lerr = P.compare_rows(wl, out, lse, q32, k32, v32, orp, oci, sample, bias=obias)
    _log(f"offset forward (oracle list), {len(sample)} sampled blocks: max|err|={err:.3e} lse {lerr:.3e}")
    assert err <= P.TOL[wl.dtype] and lerr <= P.LSE_TOL[wl.dtype]


@pytest.mark.timeout(600)
def test_ibcs_full_size_480p():
    """The clustering selector at full size (480p grid, threshold 0.9): every row's block
    list against the oracle under the same comparison rule as the small cases."""
    from oracle import ibcs
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a ROCm GPU")
    wl = WORKLOADS["wan13b_480p"]
    _log(f"[case] IBCS {wl.name} thr {wl.threshold}")
    q, k, _, _ = make_inputs(wl, "A")
    qd, kd = P.to_device(q, k)
    rp, ci = B.sparse_attn_select_ibcs(P.shape_for(wl), qd, kd, threshold=float(np.float32(wl.threshold)))
    torch.cuda.synchronize()
    rp_h = rp.cpu().numpy().astype(np.int64)
    gmask = P.check_csr(rp_h, ci[:int(rp_h[-1])].cpu().numpy(), wl.blocks)
    thr = float(np.float32(wl.threshold))
    keep, _, _, pt, gaps = ibcs.select_ibcs(q.float().numpy(), k.float().numpy(), wl.heads, thr)
    nB = wl.blocks
    rows = np.arange(wl.heads * nB)
    skip = gaps.reshape(-1)[(rows % nB) // 2 + (rows // nB) * ((nB + 1) // 2)] < P.IBCS_GAP
    ndiff, nexc, nunx = P.compare_cdf_rows(gmask, keep, pt, np.full(len(keep), thr), skip)
    _log(f"IBCS: kept {int(gmask.sum())} (oracle {int(keep.sum())}), differing {ndiff}, excused {nexc}, "
         f"unexcused {nunx}, near-tie rows {int(skip.sum())} (differing there {int((gmask[skip] != keep[skip]).sum())})")
    assert nunx == 0
    mass = (pt * gmask).sum(axis=1)
    assert np.all(mass[~skip] >= thr - 1e-4) and np.all(mass[skip] >= thr - 1e-3)
