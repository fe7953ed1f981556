"""Benchmark of the block-sparse attention hot path on one MI355X.

A step is one pass of the whole path over one batch of synthetic input:
sparse_attn_select (pooling, pooled softmax, CDF cut, CSR) followed by
sparse_attn_forward (block-sparse flash attention over the kept tiles).
The default workload is the largest configuration, the long-video layer:
batch 1, 12 heads, d=128, bf16, grid 64x48x80 (245,760 tokens, 3,840 blocks
of 1x8x8), per-head thresholds U(0.6, 0.8), inputs from the seeded generator
(reading A).  --workload picks another one.

Prints one JSON line.  `value` is the effective TFLOP/s of the whole step on
kept tiles, 4*64*64*d*nnz / t_step.  `roofline` is for the attention
kernel (MFMA bound, bf16 dense peak 2.5 PFLOP/s), its launch duration taken
with HIP events on the stream it runs on.  `cpu_baseline` times the CPU
oracle on a bounded sample of the same workload.

    python bench.py [--gpus 1] [--steps 20] [--warmup 5] [--no-cpu-baseline]
    python bench.py --pmc-summary DIR --workload W   # HBM traffic from rocprofv3 --pmc runs
    python bench.py --trace-summary DIR --steps K --warmup W   # kernel durations from a --kernel-trace run
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E
PROFILES = os.path.join(ROOT, "profiles")
CSRC = os.path.join(ROOT, "block_sparse_attention_row_amd", "csrc")
ATTN_SRC = os.path.join(CSRC, "attention.hip")
SEL_SRC = os.path.join(CSRC, "select.hip")
ATTN_KERNEL = "attn_bf16_kernel"
COPY_BYTES = 1 << 30
DEFAULT_WORKLOAD = "long_video"


def traffic_file(workload):
    return os.path.join(PROFILES, f"traffic_{workload}.json")


def _sha(path):
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--reading", default="A")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="target oracle sample time")
    ap.add_argument("--no-dense", action="store_true", help="skip the dense-CSR reference forward")
    ap.add_argument("--no-backward", action="store_true", help="skip the backward timing")
    ap.add_argument("--no-sip", action="store_true", help="skip the sampling-selection timing")
    ap.add_argument("--no-ibcs", action="store_true", help="skip the clustering-selector timing")
    ap.add_argument("--no-fine", action="store_true",
                    help="skip the 4-token key-block path (selection and gathered forward, 480p-sized inputs)")
    ap.add_argument("--sip-budget", type=float, default=0.1,
                    help="sampling selection: expected kept key blocks per row, as a fraction of the blocks")
    ap.add_argument("--no-select-timing", action="store_true", help="skip the separate selection timing")
    ap.add_argument("--dense-steps", type=int, default=0,
                    help="denoising schedule: this many leading steps run dense (no selection)")
    ap.add_argument("--reselect-every", type=int, default=1,
                    help="denoising schedule: select every K steps and reuse the block list in between")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB read + 1 GiB write kernel (torch.neg) for rocprofv3 counter scaling")
    ap.add_argument("--pmc-summary", metavar="DIR", help="summarise rocprofv3 --pmc output and exit")
    ap.add_argument("--trace-summary", metavar="DIR", help="summarise a rocprofv3 --kernel-trace run and exit")
    return ap.parse_args()


# ---------------------------------------------------------------------------- counters

def kernel_ident(name):
    """The kernel's function name, from a demangled ("void ns::name<...>(...)") or an
    Itanium-mangled ("_ZN5sattn11pool_kernelI...") kernel name."""
    if name.startswith("_ZN"):
        i, ident = 3, None
        while i < len(name) and name[i].isdigit():
            j = i
            while j < len(name) and name[j].isdigit():
                j += 1
            n = int(name[i:j])
            ident, i = name[j:j + n], j + n
        return ident
    head = name.split("<")[0].split("(")[0].split("::")[-1].split()
    return head[-1] if head else ""


def template_args(name):
    """Integer and boolean template arguments of a kernel name, in order (demangled or
    mangled: Li<n>E and Lb<0|1>E)."""
    if name.startswith("_ZN"):
        return [int(v) for v in re.findall(r"L[ib](\d+)E", name)]
    inner = name.split("<", 1)[1].rsplit(">", 1)[0] if "<" in name else ""
    out = []
    for a in inner.split(","):
        a = a.strip()
        if a in ("true", "false"):
            out.append(1 if a == "true" else 0)
        elif a.lstrip("-").isdigit():
            out.append(int(a))
    return out


def is_plain_attention(name):
    """The plain bf16 attention kernel: attn_bf16_kernel<D, ...> with every flag after D
    false (no logit offsets, no 4-token gather, no partial-tile masking)."""
    if kernel_ident(name) != ATTN_KERNEL:
        return False
    return all(v == 0 for v in template_args(name)[1:])


def is_cdf_selection(name):
    """select_emit_kernel<T, D, NE, 0>: NABLA's CDF selection (MODE 0)."""
    args = template_args(name)
    return kernel_ident(name) == "select_emit_kernel" and bool(args) and args[-1] == 0


def _read_counter_csv(pattern, counter):
    """Per-dispatch counter values by kernel name from rocprofv3 counter_collection.csv files."""
    out = {}
    for path in glob.glob(pattern, recursive=True):
        with open(path) as f:
            for row in csv.DictReader(f):
                if row.get("Counter_Name") != counter:
                    continue
                name = row.get("Kernel_Name", "")
                out.setdefault(name, []).append(float(row["Counter_Value"]))
    return out


def pmc_summary(d, workload):
    """FETCH_SIZE / WRITE_SIZE (KiB per dispatch) of the attention and selection kernels,
    scaled by what the same counters read for a plain 1 GiB copy."""
    fetch = _read_counter_csv(os.path.join(d, "fetch", "**", "*counter_collection.csv"), "FETCH_SIZE")
    write = _read_counter_csv(os.path.join(d, "write", "**", "*counter_collection.csv"), "WRITE_SIZE")

    def pick(table, match):
        vals = [v for n, vs in table.items() if match(n) for v in vs]
        return sum(vals) / len(vals) if vals else None

    def is_copy(n):                    # torch.neg over COPY_BYTES: reads and writes COPY_BYTES once
        return "neg_kernel" in n
    cf, cw = pick(fetch, is_copy), pick(write, is_copy)
    kib = COPY_BYTES / 1024.0
    fs = (kib / cf) if cf else None
    ws = (kib / cw) if cw else None
    rec = {"workload": workload, "copy_fetch_kib": cf, "copy_write_kib": cw, "copy_expected_kib": kib,
           "fetch_scale": fs, "write_scale": ws,
           "attention_source_sha256": _sha(ATTN_SRC), "selection_source_sha256": _sha(SEL_SRC), "kernels": {}}
    # the plain attention kernel (the instantiation with logit offsets serves other calls), the key
    # pooling and the CDF selection (MODE 0 of select_emit_kernel)
    for label, match in ((ATTN_KERNEL, is_plain_attention), ("pool_kernel", lambda n: kernel_ident(n) == "pool_kernel"),
                         ("select_emit_kernel", is_cdf_selection)):
        f, w = pick(fetch, match), pick(write, match)
        k = {"fetch_kib_per_dispatch": f, "write_kib_per_dispatch": w}
        if f and w and fs and ws:
            k["hbm_bytes_per_dispatch"] = f * 1024.0 * fs + w * 1024.0 * ws
        rec["kernels"][label] = k
    print(json.dumps(rec, indent=1))
    return rec


def stored_traffic(workload):
    """(attention bytes, selection bytes) per launch from the stored counter summary, or
    None for each when absent or taken on a different kernel source."""
    try:
        rec = json.load(open(traffic_file(workload)))
    except (OSError, ValueError):
        return None, None
    if rec.get("workload") != workload:
        return None, None
    ks = rec.get("kernels", {})
    attn = ks.get(ATTN_KERNEL, {}).get("hbm_bytes_per_dispatch")
    if rec.get("attention_source_sha256") != _sha(ATTN_SRC):
        attn = None            # the kernel changed since the counters were taken
    sel = None
    if rec.get("selection_source_sha256") == _sha(SEL_SRC):
        a = ks.get("pool_kernel", {}).get("hbm_bytes_per_dispatch")
        b = ks.get("select_emit_kernel", {}).get("hbm_bytes_per_dispatch")
        sel = (a + b) if (a and b) else None
    return attn, sel


def trace_summary(d, steps, warmup):
    """Per-kernel durations from rocprofv3 --kernel-trace CSV files, as a markdown table;
    for the attention kernel also the dispatches of the timed steps alone (the plain
    kernel's dispatches warmup .. warmup + steps - 1: bench.py's warm-up steps come
    first and the timed steps next)."""
    rows = []
    for path in glob.glob(os.path.join(d, "**", "*kernel_trace.csv"), recursive=True):
        with open(path) as f:
            for r in csv.DictReader(f):
                rows.append((int(r["Start_Timestamp"]), int(r["End_Timestamp"]), r["Kernel_Name"]))
    rows.sort()
    by = {}
    for t0, t1, name in rows:
        by.setdefault(name, []).append((t1 - t0) / 1000.0)

    def stats(v):
        s = sorted(v)
        return len(v), sum(v) / len(v), s[len(s) // 2], s[0], s[-1], sum(v) / 1000.0
    out = ["| kernel | calls | avg us | median us | min us | max us | total ms |", "|---|---|---|---|---|---|---|"]
    for name, v in sorted(by.items(), key=lambda kv: -sum(kv[1])):
        n, a, m, lo, hi, tot = stats(v)
        short = name.split("(")[0][:90]
        out.append(f"| `{short}` | {n} | {a:.1f} | {m:.1f} | {lo:.1f} | {hi:.1f} | {tot:.2f} |")
    plain = [v for name, v in by.items() if is_plain_attention(name)]
    if plain:
        timed = plain[0][warmup:warmup + steps]
        if timed:
            n, a, m, lo, hi, _ = stats(timed)
            out.append("")
            out.append(f"Timed steps only (`{ATTN_KERNEL}`, plain, dispatches {warmup} .. {warmup + steps - 1}): "
                       f"{n} calls, avg {a:.1f} us, median {m:.1f} us, min {lo:.1f} us, max {hi:.1f} us.")
    print("\n".join(out))


# ---------------------------------------------------------------------------- GPU bench

def main():
    args = parse()
    if args.pmc_summary:
        pmc_summary(args.pmc_summary, args.workload)
        return
    if args.trace_summary:
        trace_summary(args.trace_summary, args.steps, args.warmup)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}); "
              "the path shards by head with no exchange, see the design notes", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from block_sparse_attention_row_amd import binding as B
    from block_sparse_attention_row_amd.synth import WORKLOADS, make_inputs

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    B.lib()
    wl = WORKLOADS[args.workload]
    t0 = time.time()
    q, k, v, thr = make_inputs(wl, args.reading)
    print(f"[bench] inputs {wl.name} reading {args.reading} drawn in {time.time() - t0:.1f}s", file=sys.stderr,
          flush=True)
    dev = torch.device("cuda:0")
    qd, kd, vd = (t.to(dev) for t in (q, k, v))
    shape = B.make_shape(wl.batch, wl.heads, wl.head_dim, wl.grid, wl.dtype, 0.0, wl.tile)
    bufs = B.alloc_buffers(shape, dev)
    out = torch.empty_like(qd)
    lse = torch.empty(qd.shape[:3], dtype=torch.float32, device=dev)
    head_thr = None if wl.head_threshold_range is None else [float(x) for x in thr]
    stream = torch.cuda.current_stream()

    def select():
        return B.sparse_attn_select(shape, qd, kd, threshold=float(np.float32(wl.threshold)),
                                    head_thresholds=head_thr, window=wl.window, buffers=bufs, stream=stream)

    def forward(rp, ci):
        B.sparse_attn_forward(shape, qd, kd, vd, rp, ci, out=out, lse=lse, workspace=bufs.workspace,
                              stream=stream)

    def step():
        rp, ci = select()
        forward(rp, ci)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    nnz = int(bufs.row_ptr[-1].item())
    rows = wl.batch * wl.heads * wl.blocks

    # timed region: exactly `steps` steps, synchronised on both sides
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for i in range(args.steps):
        rp, ci = select()
        ev[i][0].record(stream)
        forward(rp, ci)
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    t_total = time.perf_counter() - t_start
    ms_step = 1000.0 * t_total / args.steps
    attn_ms = [a.elapsed_time(b) for a, b in ev]
    attn_ms_avg = sum(attn_ms) / len(attn_ms)

    flops = 4.0 * 64 * 64 * wl.head_dim * nnz
    value = flops / (ms_step * 1e-3) / 1e12
    attn_tflops = flops / (attn_ms_avg * 1e-3) / 1e12

    # selection alone, each repetition after a read-only 1 GiB sweep, so that Q and K do
    # not sit in the last-level cache and no dirty lines are left to write back
    flush = torch.ones(1 << 28, dtype=torch.float32, device=dev)
    sel_ms = []
    for _ in range(0 if args.no_select_timing else 10):
        flush.sum()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        select()
        b.record(stream)
        torch.cuda.synchronize()
        sel_ms.append(a.elapsed_time(b))
    sel_ms_med = sorted(sel_ms)[len(sel_ms) // 2] if sel_ms else float("nan")
    elt = qd.element_size()
    sel_bytes = 2 * qd.numel() * elt + 4 * (rows + 1) + 4 * nnz
    sel_gbs = sel_bytes / (sel_ms_med * 1e-3) / 1e9

    # token reordering raster -> tile-major of Q (a data-movement kernel: read + write)
    reo = torch.empty_like(qd)
    reo_ms = []
    for _ in range(0 if args.no_select_timing else 5):
        flush.sum()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        B.sparse_attn_to_tiles(shape, qd, reo, stream=stream)
        b.record(stream)
        torch.cuda.synchronize()
        reo_ms.append(a.elapsed_time(b))
    reo_ms_med = sorted(reo_ms)[len(reo_ms) // 2] if reo_ms else float("nan")
    reo_gbs = 2 * qd.numel() * elt / (reo_ms_med * 1e-3) / 1e9
    del reo

    # raster-ordered Q and K: the two reorders followed by the selection, against the
    # selection on raster inputs with the reorder fused into the pooling (same block
    # list and tile-major copies); interleaved repetitions, each after the sweep
    raster = None
    if not args.no_select_timing:
        qr = B.sparse_attn_from_tiles(shape, qd, stream=stream)
        kr = B.sparse_attn_from_tiles(shape, kd, stream=stream)
        qt, kt = torch.empty_like(qd), torch.empty_like(kd)
        rbufs = B.alloc_buffers(shape, dev)
        kw = dict(threshold=float(np.float32(wl.threshold)), head_thresholds=head_thr, window=wl.window,
                  buffers=rbufs, stream=stream)

        def separate():
            B.sparse_attn_to_tiles(shape, qr, qt, stream=stream)
            B.sparse_attn_to_tiles(shape, kr, kt, stream=stream)
            B.sparse_attn_select(shape, qt, kt, **kw)

        def fused():
            B.sparse_attn_select_raster(shape, qr, kr, qt, kt, **kw)
        times = {"separate": [], "fused": []}
        for _ in range(7):
            for name, fn in (("separate", separate), ("fused", fused)):
                flush.sum()
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record(stream)
                fn()
                b.record(stream)
                torch.cuda.synchronize()
                times[name].append(a.elapsed_time(b))
        med = {n: sorted(v)[len(v) // 2] for n, v in times.items()}
        r_bytes = 4 * qd.numel() * elt + 4 * (rows + 1) + 4 * nnz      # Q, K read and written, CSR
        r_gbs = r_bytes / (med["fused"] * 1e-3) / 1e9
        raster = {"reorder_then_select_ms": round(med["separate"], 4), "fused_ms": round(med["fused"], 4),
                  "bytes": r_bytes, "fused_GB_s": round(r_gbs, 1), "fused_frac_hbm_peak": round(r_gbs / PEAK_HBM_GBS, 4)}
        del qr, kr, qt, kt, rbufs

    # backward over the selected block list (bf16): dQ over the rows, dK and dV over the
    # transposed list; FLOPs counted as the five algorithmic products (S, dP, dV, dQ, dK)
    bwd = None
    if wl.dtype == "bf16" and not args.no_backward:
        rp, ci = select()
        forward(rp, ci)
        ci = ci[:nnz]                      # the backward's transposed list holds one entry per listed one
        gen = torch.Generator(device=dev).manual_seed(5)
        dout = torch.randn(qd.shape, generator=gen, device=dev).to(qd.dtype)
        grads = tuple(torch.empty_like(qd) for _ in range(3))
        t_idx = torch.empty(max(nnz, 1), dtype=torch.int32, device=dev)

        def backward():
            B.sparse_attn_backward(shape, qd, kd, vd, out, lse, dout, rp, ci, workspace=bufs.workspace,
                                   t_idx=t_idx, stream=stream, grads=grads)
        backward()
        bwd_ms = []
        for _ in range(5):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            backward()
            b.record(stream)
            torch.cuda.synchronize()
            bwd_ms.append(a.elapsed_time(b))
        bwd_ms_med = sorted(bwd_ms)[len(bwd_ms) // 2]
        bwd_tf = 2.5 * flops / (bwd_ms_med * 1e-3) / 1e12
        bwd = {"ms": round(bwd_ms_med, 4), "TFLOP_s": round(bwd_tf, 2),
               "frac_bf16_peak": round(bwd_tf / PEAK_BF16_TFLOPS, 4)}
        del dout, grads, t_idx

    # sampling with inclusion probabilities (AB-Attention's SIP) on the same inputs: the
    # selection (after the cache sweep, like the CDF selection) and the forward with
    # the Horvitz-Thompson logit offsets over the sampled list
    sip = None
    if wl.dtype == "bf16" and not args.no_sip:
        budget = args.sip_budget * wl.blocks
        sbufs = B.alloc_buffers(shape, dev)
        cbias = torch.empty(sbufs.col_idx.numel(), dtype=torch.float32, device=dev)

        def sip_select():
            return B.sparse_attn_select_sip(shape, qd, kd, budget, seed=2026, buffers=sbufs, col_bias=cbias,
                                            stream=stream)
        srp, sci, _ = sip_select()
        torch.cuda.synchronize()
        snnz = int(srp[-1].item())
        sip_ms = []
        for _ in range(10):
            flush.sum()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            sip_select()
            b.record(stream)
            torch.cuda.synchronize()
            sip_ms.append(a.elapsed_time(b))
        sip_ms_med = sorted(sip_ms)[len(sip_ms) // 2]
        sip_bytes = 2 * qd.numel() * elt + 4 * (rows + 1) + 8 * snnz
        for _ in range(2):
            B.sparse_attn_forward_biased(shape, qd, kd, vd, srp, sci, cbias, out=out, lse=lse,
                                         workspace=bufs.workspace, stream=stream)
        fw_ms = []
        for _ in range(10):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            B.sparse_attn_forward_biased(shape, qd, kd, vd, srp, sci, cbias, out=out, lse=lse,
                                         workspace=bufs.workspace, stream=stream)
            b.record(stream)
            torch.cuda.synchronize()
            fw_ms.append(a.elapsed_time(b))
        fw_ms_med = sorted(fw_ms)[len(fw_ms) // 2]
        sip_flops = 4.0 * 64 * 64 * wl.head_dim * snnz
        sip = {"budget_blocks_per_row": budget, "nnz_tiles": snnz, "kept_fraction": round(snnz / (rows * wl.blocks), 4),
               "select_ms": round(sip_ms_med, 4), "select_GB_s": round(sip_bytes / (sip_ms_med * 1e-3) / 1e9, 1),
               "select_frac_hbm_peak": round(sip_bytes / (sip_ms_med * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
               "forward_ms": round(fw_ms_med, 4),
               "forward_TFLOP_s": round(sip_flops / (fw_ms_med * 1e-3) / 1e12, 2),
               "forward_frac_bf16_peak": round(sip_flops / (fw_ms_med * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)}
        del sbufs, cbias

    # clustering selector (AB-Attention's IBCS) with NABLA's CDF cut, same threshold
    ibcs = None
    if wl.dtype == "bf16" and not args.no_ibcs:
        ibufs = B.alloc_buffers(shape, dev)

        def ibcs_select():
            return B.sparse_attn_select_ibcs(shape, qd, kd, threshold=float(np.float32(wl.threshold)),
                                             head_thresholds=head_thr, window=wl.window, buffers=ibufs,
                                             stream=stream)
        irp, _ = ibcs_select()
        torch.cuda.synchronize()
        innz = int(irp[-1].item())
        ims = []
        for _ in range(5):
            flush.sum()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            ibcs_select()
            b.record(stream)
            torch.cuda.synchronize()
            ims.append(a.elapsed_time(b))
        ims_med = sorted(ims)[len(ims) // 2]
        ibytes = 2 * qd.numel() * elt + 4 * (rows + 1) + 4 * innz
        ibcs = {"ms": round(ims_med, 4), "nnz_tiles": innz, "GB_s": round(ibytes / (ims_med * 1e-3) / 1e9, 1),
                "frac_hbm_peak": round(ibytes / (ims_med * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}
        del ibufs

    # AB-Attention's 4-token key blocks: the selection over 16 nB key blocks a row and the
    # forward that gathers the kept blocks into tiles, on the 480p-sized workload (the
    # 4-token selection serves rows of up to 512 query blocks)
    fine = None
    if not args.no_fine:
        fwl = WORKLOADS["wan13b_480p"]
        fq, fk, fv, _ = make_inputs(fwl, args.reading)
        fqd, fkd, fvd = fq.to(dev), fk.to(dev), fv.to(dev)
        del fq, fk, fv
        fshape = B.make_shape(fwl.batch, fwl.heads, fwl.head_dim, fwl.grid, fwl.dtype, 0.0, fwl.tile)
        fthr = float(np.float32(fwl.threshold))
        fws = torch.empty(B.sparse_attn_fine_workspace_size(fshape), dtype=torch.uint8, device=dev)
        frows = fwl.batch * fwl.heads * fwl.blocks
        frp = torch.empty(frows + 1, dtype=torch.int32, device=dev)
        fci = torch.empty(B.sparse_attn_fine_csr_capacity(fshape), dtype=torch.int32, device=dev)
        fout = torch.empty_like(fqd)
        fwsa = torch.empty(B.sparse_attn_workspace_size(fshape), dtype=torch.uint8, device=dev)

        def fine_select():
            return B.sparse_attn_select_fine(fshape, fqd, fkd, threshold=fthr, row_ptr=frp, col_idx=fci,
                                             workspace=fws, stream=stream)

        def fine_forward():
            B.sparse_attn_forward_gather(fshape, fqd, fkd, fvd, frp, fci, out=fout, workspace=fwsa, stream=stream)
        fine_select()
        fine_forward()
        torch.cuda.synchronize()
        fnnz = int(frp[-1].item())
        fsel, ffw = [], []
        for _ in range(10):
            flush.sum()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            fine_select()
            b.record(stream)
            torch.cuda.synchronize()
            fsel.append(a.elapsed_time(b))
        for _ in range(10):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            fine_forward()
            b.record(stream)
            torch.cuda.synchronize()
            ffw.append(a.elapsed_time(b))
        fsel_med, ffw_med = sorted(fsel)[5], sorted(ffw)[5]
        nK = 16 * fwl.blocks
        fbytes = 2 * fqd.numel() * fqd.element_size() + 4 * (frows + 1) + 4 * fnnz
        fflops = 4.0 * 64 * 4 * fwl.head_dim * fnnz        # 64 queries x 4 keys per kept block
        fine = {"workload": fwl.name, "key_blocks_per_row": nK, "nnz_key_blocks": fnnz,
                "kept_fraction": round(fnnz / (frows * nK), 4),
                "select_ms": round(fsel_med, 4), "select_GB_s": round(fbytes / (fsel_med * 1e-3) / 1e9, 1),
                "select_frac_hbm_peak": round(fbytes / (fsel_med * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                "forward_ms": round(ffw_med, 4),
                "forward_TFLOP_s": round(fflops / (ffw_med * 1e-3) / 1e12, 2),
                "forward_frac_bf16_peak": round(fflops / (ffw_med * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)}
        del fqd, fkd, fvd, fws, fci, fout, fwsa

    # dense reference: the same forward kernel over the full CSR (every tile kept)
    full_bufs = B.alloc_buffers(shape, dev)
    full_rp, full_ci = B.sparse_attn_full_csr(shape, full_bufs, stream=stream)
    for _ in range(0 if args.no_dense else 2):
        B.sparse_attn_forward(shape, qd, kd, vd, full_rp, full_ci, out=out, lse=lse, workspace=bufs.workspace,
                              stream=stream)
    dense_ms = []
    for _ in range(0 if args.no_dense else 5):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        B.sparse_attn_forward(shape, qd, kd, vd, full_rp, full_ci, out=out, lse=lse, workspace=bufs.workspace,
                              stream=stream)
        b.record(stream)
        torch.cuda.synchronize()
        dense_ms.append(a.elapsed_time(b))
    dense_ms_med = sorted(dense_ms)[len(dense_ms) // 2] if dense_ms else float("nan")

    if args.copy_calibration:
        src = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        for _ in range(2):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        del src, dst

    # optional denoising schedule: dense warm-up steps, then a selection every K steps
    # whose block list the steps in between reuse
    sched = None
    if args.dense_steps > 0 or args.reselect_every > 1:
        K = max(1, args.reselect_every)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        tiles = 0
        rp_s, ci_s = None, None
        for i in range(args.steps):
            if i < args.dense_steps:
                forward(full_rp, full_ci)
                tiles += rows * wl.blocks
            else:
                if (i - args.dense_steps) % K == 0:
                    rp_s, ci_s = select()
                forward(rp_s, ci_s)
                tiles += nnz
        torch.cuda.synchronize()
        t_s = (time.perf_counter() - t0) / args.steps
        sched = {"dense_steps": args.dense_steps, "reselect_every": K, "ms_per_step": round(1e3 * t_s, 4),
                 "TFLOP_s": round(4.0 * 64 * 64 * wl.head_dim * tiles / args.steps / t_s / 1e12, 2)}

    traffic, sel_traffic = stored_traffic(wl.name)
    rec = {
        "metric": "effective TFLOP/s on kept tiles (select + forward step)",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if wl.dtype == "bf16" else "f32",
        "data": "synthetic (seeded smoothed-Gaussian Q, K = Q + noise, Gaussian V)",
        "config": {
            "workload": wl.name, "batch": wl.batch, "heads": wl.heads, "head_dim": wl.head_dim,
            "grid": list(wl.grid), "tokens": wl.tokens, "blocks": wl.blocks, "threshold": wl.threshold,
            "window": list(wl.window), "reading": args.reading, "nnz_tiles": nnz,
            "kept_fraction": round(nnz / (rows * wl.blocks), 4),
        },
        "roofline": {
            "bound": "mfma", "achieved": round(attn_tflops, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
            "frac": round(attn_tflops / PEAK_BF16_TFLOPS, 4), "traffic": traffic,
            "kernel": ATTN_KERNEL, "launch_ms": round(attn_ms_avg, 4),
            "flops_per_launch": flops,
        },
        "attention_tflops_pct_peak": round(100 * attn_tflops / PEAK_BF16_TFLOPS, 2),
        "selection": {
            "ms": round(sel_ms_med, 4), "bytes": sel_bytes, "GB_s": round(sel_gbs, 1),
            "frac_hbm_peak": round(sel_gbs / PEAK_HBM_GBS, 4), "traffic": sel_traffic,
        },
        "reorder_to_tiles": {"ms": round(reo_ms_med, 4), "GB_s": round(reo_gbs, 1),
                             "frac_hbm_peak": round(reo_gbs / PEAK_HBM_GBS, 4)},
        "raster_select": raster,
        "dense_forward_ms": round(dense_ms_med, 4),
        "speedup_vs_dense": {
            "forward": round(dense_ms_med / attn_ms_avg, 3),
            "select_plus_forward": round(dense_ms_med / (attn_ms_avg + sel_ms_med), 3),
        },
    }
    if bwd is not None:
        rec["backward"] = bwd
    if sip is not None:
        rec["sip"] = sip
    if ibcs is not None:
        rec["ibcs"] = ibcs
    if fine is not None:
        rec["fine_4token"] = fine
    if sched is not None:
        rec["denoise_schedule"] = sched
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(wl, q, k, v, thr, bufs, args.cpu_seconds)
    print(json.dumps(rec), flush=True)


def _host_info():
    try:
        n_aff = len(os.sched_getaffinity(0))
    except AttributeError:
        n_aff = os.cpu_count() or 1
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    omp = os.environ.get("OMP_NUM_THREADS")
    threads = int(omp) if omp and omp.isdigit() else n_aff
    return {"nproc": n_aff, "cpu_model": model, "omp_num_threads": omp, "threads": threads}


def sample_blocks(wl, thr, n_heads=2, n_blocks=32, seed=1):
    """The oracle's sample: 2 heads x 32 query blocks drawn with rng(1); with per-head
    thresholds, the heads of the lowest and the highest threshold."""
    import numpy as np
    rng = np.random.default_rng(seed)
    if wl.head_threshold_range is not None:
        heads = [int(np.argmin(thr)), int(np.argmax(thr))]
    else:
        heads = sorted(rng.choice(wl.heads, size=min(n_heads, wl.heads), replace=False).tolist())
    rows = []
    for h in heads:
        blocks = np.sort(rng.choice(wl.blocks, size=min(n_blocks, wl.blocks), replace=False))
        rows.extend((h * wl.blocks + blocks).tolist())        # batch 0
    return np.array(rows, dtype=np.int64), heads


def cpu_baseline(wl, q, k, v, thr, bufs, target_s):
    """The CPU oracle, as it stands, on the host cores of the GPU machine (rank 0, one GPU):
    the whole selection (pooling, pooled softmax, CDF cut, window) on every row, and the
    attention of a sample of query blocks (2 heads x 32 blocks, rng(1)) under the GPU's
    block list; the per-block time extrapolated to the whole step, labelled as such."""
    import numpy as np
    import oracle
    host = _host_info()
    rows = wl.batch * wl.heads * wl.blocks
    rp = bufs.row_ptr.cpu().numpy().astype(np.int64)
    ci = bufs.col_idx[:int(rp[-1])].cpu().numpy()
    q32, k32 = q.float().numpy(), k.float().numpy()
    t0 = time.perf_counter()
    qbar, kbar = oracle.pool(q32), oracle.pool(k32)
    oracle.select_rows(qbar, kbar, wl.heads, wl.block_grid, thr.astype(np.float64), wl.window)
    t_sel = time.perf_counter() - t0
    del q32, k32
    sample, heads = sample_blocks(wl, thr)
    t0 = time.perf_counter()
    oracle.attention_rows(q, k, v, rp, ci, sample)
    t = time.perf_counter() - t0
    tiles = int(np.sum(rp[sample + 1] - rp[sample]))
    tflops = 4.0 * 64 * 64 * wl.head_dim * tiles / t / 1e12
    per_block = t / len(sample)
    # the full step extrapolated by kept tiles (rows differ in length across heads)
    full_attn = t * float(rp[-1]) / max(tiles, 1)
    return {"value": tflops, "unit": "TFLOP/s", "cores": host["threads"], "kind": "oracle",
            "sample": f"fp64 oracle: full selection of all {rows} query blocks ({t_sel:.1f} s); attention of "
                      f"{len(sample)} query blocks (heads {heads} x 32 blocks, rng(1); {tiles} kept tiles, "
                      f"{t:.1f} s) under the GPU's block list",
            "selection_s": round(t_sel, 3), "attention_s_per_query_block": round(per_block, 4),
            "extrapolated_full_step_s": round(t_sel + full_attn, 1),
            "extrapolation": "selection measured in full; attention scaled from the sample by kept tiles",
            **host}


if __name__ == "__main__":
    main()
