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
    attn = "void sattn::attn_bf16_kernel<128, false>(sattn::AttnArgs)"
    biased = "void sattn::attn_bf16_kernel<128, true>(sattn::AttnArgs)"
    copy = "void at::native::vectorized_elementwise_kernel<4, neg_kernel>"
    # the copy reads and writes 1 GiB but the counters read half of it on fetch
    _write_counters(str(tmp_path / "fetch" / "a" / "run_counter_collection.csv"), "FETCH_SIZE",
                    [(copy, kib / 2), (attn, 1000.0), (attn, 1200.0), (biased, 9.0e9)])
    _write_counters(str(tmp_path / "write" / "a" / "run_counter_collection.csv"), "WRITE_SIZE",
                    [(copy, kib), (attn, 300.0), (attn, 300.0), (biased, 9.0e9)])
    rec = bench.pmc_summary(str(tmp_path))
    assert rec["fetch_scale"] == pytest.approx(2.0)
    assert rec["write_scale"] == pytest.approx(1.0)
    # the plain kernel's dispatches only, averaged, in bytes
    assert rec["hbm_bytes_per_dispatch"] == pytest.approx(1100.0 * 1024 * 2.0 + 300.0 * 1024)


def test_stored_traffic_needs_the_same_source_and_workload(tmp_path, monkeypatch):
    src = tmp_path / "attention.hip"
    src.write_text("// kernel v1\n")
    rec = {"attention_source_sha256": hashlib.sha256(src.read_bytes()).hexdigest(), "workload": "wan13b_480p",
           "hbm_bytes_per_dispatch": 123.0}
    tf = tmp_path / "traffic.json"
    tf.write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "ATTN_SRC", str(src))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tf))
    assert bench.stored_traffic("wan13b_480p") == 123.0
    assert bench.stored_traffic("long_video") is None         # counters of another workload
    src.write_text("// kernel v2\n")
    assert bench.stored_traffic("wan13b_480p") is None        # kernel changed since the counters
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "missing.json"))
    assert bench.stored_traffic("wan13b_480p") is None


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
