"""Host-side logic with no GPU: bench.py's one-GPU guard, its HBM-traffic record and
the check that ties a stored traffic figure to its kernel source and workload, and
the forward's query-block pairing as mirrored by the tests."""
import csv
import hashlib
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def _write_counters(path, counter, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for i, (name, value) in enumerate(rows):
            w.writerow({"Dispatch_Id": i, "Kernel_Name": name, "Counter_Name": counter, "Counter_Value": value})


def test_pmc_summary_scales_by_the_copy_kernel(tmp_path):
    kib = bench.COPY_BYTES / 1024.0
    attn = "void sattn::attn_bf16_kernel<128, false, false, false>(sattn::AttnArgs)"
    biased = "void sattn::attn_bf16_kernel<128, true, false, false>(sattn::AttnArgs)"
    gathered = "void sattn::attn_bf16_kernel<128, false, true, false>(sattn::AttnArgs)"
    fine_pool = "_ZN5sattn16fine_pool_kernelILi128EEEvPKDF16bPfS3_llNS_8PoolSideE"     # not the key pooling
    sel_mangled = "_ZN5sattn18select_emit_kernelIDF16bLi128ELi60ELi0EEEvNS_10SelectArgsE"
    pool = "void sattn::pool_kernel<__bf16, 128>(__bf16 const*, __bf16*, long, int, sattn::PoolSide)"
    sel = "sattn::select_emit_kernel<bf16, 128, 60, 0>"
    sip = "sattn::select_emit_kernel<bf16, 128, 60, 1>"
    copy = "void at::native::vectorized_elementwise_kernel<4, neg_kernel>"
    # the copy reads and writes 1 GiB but the counters read half of it on fetch
    _write_counters(str(tmp_path / "fetch" / "a" / "run_counter_collection.csv"), "FETCH_SIZE",
                    [(copy, kib / 2), (attn, 1000.0), (attn, 1200.0), (biased, 9.0e9), (gathered, 9.0e9),
                     (pool, 50.0), (fine_pool, 9.0e9), (sel, 70.0), (sel_mangled, 70.0), (sip, 9.0e9)])
    _write_counters(str(tmp_path / "write" / "a" / "run_counter_collection.csv"), "WRITE_SIZE",
                    [(copy, kib), (attn, 300.0), (attn, 300.0), (biased, 9.0e9), (gathered, 9.0e9), (pool, 5.0),
                     (fine_pool, 9.0e9), (sel, 7.0), (sel_mangled, 7.0), (sip, 9.0e9)])
    rec = bench.pmc_summary(str(tmp_path), "long_video")
    assert rec["fetch_scale"] == pytest.approx(2.0)
    assert rec["write_scale"] == pytest.approx(1.0)
    # the plain kernel's dispatches only, averaged, in bytes
    k = rec["kernels"]
    assert k["attn_bf16_kernel"]["hbm_bytes_per_dispatch"] == pytest.approx(1100.0 * 1024 * 2.0 + 300.0 * 1024)
    # the CDF selection (MODE 0) only, not the sampling selection
    assert k["select_emit_kernel"]["hbm_bytes_per_dispatch"] == pytest.approx(70.0 * 1024 * 2.0 + 7.0 * 1024)
    assert k["pool_kernel"]["hbm_bytes_per_dispatch"] == pytest.approx(50.0 * 1024 * 2.0 + 5.0 * 1024)


def test_stored_traffic_needs_the_same_source_and_workload(tmp_path, monkeypatch):
    src = tmp_path / "attention.hip"
    src.write_text("// kernel v1\n")
    sel_src = tmp_path / "select.hip"
    sel_src.write_text("// selection v1\n")
    sha = lambda p: hashlib.sha256(p.read_bytes()).hexdigest()
    rec = {"attention_source_sha256": sha(src), "selection_source_sha256": sha(sel_src), "workload": "long_video",
           "kernels": {"attn_bf16_kernel": {"hbm_bytes_per_dispatch": 123.0},
                       "pool_kernel": {"hbm_bytes_per_dispatch": 10.0},
                       "select_emit_kernel": {"hbm_bytes_per_dispatch": 20.0}}}
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    (tmp_path / "traffic_long_video.json").write_text(json.dumps(rec))
    (tmp_path / "traffic_wan13b_480p.json").write_text(json.dumps(rec))     # names another workload inside
    monkeypatch.setattr(bench, "ATTN_SRC", str(src))
    monkeypatch.setattr(bench, "SEL_SRC", str(sel_src))
    assert bench.stored_traffic("long_video") == (123.0, 30.0)
    assert bench.stored_traffic("wan13b_480p") == (None, None)       # counters of another workload
    src.write_text("// kernel v2\n")
    assert bench.stored_traffic("long_video") == (None, 30.0)        # attention changed since the counters
    sel_src.write_text("// selection v2\n")
    assert bench.stored_traffic("long_video") == (None, None)
    assert bench.stored_traffic("hunyuan_720p") == (None, None)      # no counters at all


def test_trace_summary_separates_the_timed_steps(tmp_path, capsys):
    path = tmp_path / "x" / "run_kernel_trace.csv"
    os.makedirs(path.parent)
    attn = "void sattn::attn_bf16_kernel<128, false, false, false>(sattn::AttnArgs)"
    biased = "void sattn::attn_bf16_kernel<128, true, false, false>(sattn::AttnArgs)"
    rows = []
    t = 0
    for i, dur_us in enumerate([900, 800, 240, 241, 239, 500]):      # 2 warm-ups, 3 timed, 1 later call
        rows.append({"Kernel_Name": attn, "Start_Timestamp": t, "End_Timestamp": t + dur_us * 1000})
        t += 10 ** 7
    for dur_us in (70, 71):                                           # the biased kernel is not the plain one
        rows.append({"Kernel_Name": biased, "Start_Timestamp": t, "End_Timestamp": t + dur_us * 1000})
        t += 10 ** 7
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Start_Timestamp", "End_Timestamp"])
        w.writeheader()
        w.writerows(rows)
    bench.trace_summary(str(tmp_path), steps=3, warmup=2)
    out = capsys.readouterr().out
    assert "3 calls, avg 240.0 us, median 240.0 us, min 239.0 us, max 241.0 us" in out


def test_plain_attention_kernel_names():
    assert bench.is_plain_attention("void sattn::attn_bf16_kernel<128, false, false, false>(sattn::AttnArgs)")
    assert bench.is_plain_attention("sattn::attn_bf16_kernel<64, false>")
    for flags in ("true, false, false", "false, true, false", "false, false, true"):
        assert not bench.is_plain_attention(f"void sattn::attn_bf16_kernel<128, {flags}>(sattn::AttnArgs)")
    assert not bench.is_plain_attention("void sattn::pool_kernel<__bf16, 128>(...)")
    # library kernels whose names carry no identifier before the parameters
    for odd in ("void at::native::(anonymous namespace)::fill_kernel(float*)", "void (anonymous)", "", "()"):
        assert not bench.is_plain_attention(odd) and not bench.is_cdf_selection(odd)


def test_cpu_baseline_sample_is_two_heads_of_32_blocks():
    import numpy as np
    from block_sparse_attention_row_amd.synth import WORKLOADS, head_thresholds
    wl = WORKLOADS["long_video"]
    thr = head_thresholds(wl)
    rows, heads = bench.sample_blocks(wl, thr)
    assert heads == [int(np.argmin(thr)), int(np.argmax(thr))]
    assert len(rows) == 64 and len(np.unique(rows)) == 64
    assert set((rows // wl.blocks).tolist()) == set(heads)
    info = bench._host_info()
    assert info["nproc"] >= 1 and info["threads"] >= 1 and info["cpu_model"]


@pytest.mark.parametrize("nt,s", [(20, 24), (21, 60), (7, 15), (3, 3), (1, 24), (480, 1), (105, 1), (2, 1)])
def test_forward_pairs_cover_every_block_once(nt, s):
    """The host mirror of the forward's query-block pairs (tests/parity.py) is a
    partition of the blocks into ceil(nB/2) pairs of frame-neighbours (side by side in
    an odd last frame)."""
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    import parity as P
    nb = nt * s
    stride = s if nt >= 2 else 1
    seen = []
    for p in range((nb + 1) // 2):
        a, b = P.pair_blocks(p, stride, nb)
        seen.append(a)
        if b >= 0:
            seen.append(b)
            assert b == a + stride or (a // stride == nt - 1 and b == a + 1)
    assert sorted(seen) == list(range(nb))
