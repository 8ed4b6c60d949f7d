"""Host logic of bench.py (no GPU): the one-GPU guard, the comment-blind source hash
that keys committed counter records, and the ingestion of rocprofv3 counter runs
(calibration against a plain copy, per-kind means, pruning of records taken on
other sources)."""
import csv
import json
import os
import subprocess
import sys

import pytest

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_code_only_ignores_comments_and_layout():
    a = 'int a = 1; // one\n/* two\n   lines */\n\n    int b = a + 2;\nconst char *s = "// kept";\n'
    b = 'int a = 1;\nint b = a + 2;\nconst char *s = "// kept";\n'
    assert bench._code_only(a) == bench._code_only(b)
    assert '"// kept"' in bench._code_only(a)
    assert bench._code_only("int a = 1;") != bench._code_only("int a = 2;")


def test_source_hash_groups():
    # decode and the token loop share one source group; the split kinds share another
    assert bench.kernel_source_hash("recurrent") != bench.kernel_source_hash("recur")
    assert bench.kernel_source_hash("prep") == bench.kernel_source_hash("recur")
    assert bench.kernel_source_hash("fused") != bench.kernel_source_hash("recur")


def _counter_csv(path, counter, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for name, kib in rows:
            w.writerow({"Kernel_Name": name, "Counter_Name": counter, "Counter_Value": kib})


def test_ingest_scales_by_the_copy_and_prunes_stale_records(tmp_path, monkeypatch):
    out = tmp_path / "traffic.json"
    # a record taken on other sources: dropped at the next ingestion
    out.write_text(json.dumps({"kernels": {"recur@old": {"source_hash": "0" * 16, "workload": "old"}}}))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(out))
    copy = "__amd_rocclr_copyBuffer"
    prep = "kda::prep_kernel(unsigned short const*, ...)"
    pair = "void kda::recur_pair_kernel<1, 5>(char const*, ...)"
    rp = "void kda::recur_prep_kernel<1, 5>(char const*, ...)"
    mib = 1024.0                                   # counters count KiB: 1 MiB = 1024
    # FETCH_SIZE counts half the bytes of the 256 MiB copy, WRITE_SIZE all of them
    _counter_csv(tmp_path / "f.csv", "FETCH_SIZE",
                 [(copy, 128 * mib), (prep, 10 * mib), (prep, 30 * mib), (pair, 5 * mib), (rp, 7 * mib)])
    _counter_csv(tmp_path / "w.csv", "WRITE_SIZE",
                 [(copy, 256 * mib), (prep, 4 * mib), (prep, 4 * mib), (pair, 1 * mib), (rp, 3 * mib)])
    bench.ingest_pmc(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"), "unit", "cmd")
    t = json.loads(out.read_text())
    assert t["fetch_scale"] == pytest.approx(2.0) and t["write_scale"] == pytest.approx(1.0)
    k = t["kernels"]
    assert set(k) == {"prep@unit", "recur@unit", "recur_prep@unit"}
    m = float(1 << 20)
    assert k["prep@unit"]["fetch_bytes"] == pytest.approx(2 * 20 * m)     # mean of 10 and 30, x2
    assert k["prep@unit"]["write_bytes"] == pytest.approx(4 * m)
    assert k["prep@unit"]["dispatches"] == 2
    assert k["recur@unit"]["bytes_per_launch"] == pytest.approx(2 * 5 * m + 1 * m)
    assert k["recur_prep@unit"]["bytes_per_launch"] == pytest.approx(2 * 7 * m + 3 * m)
    assert all(r["source_hash"] == bench.kernel_source_hash(name.split("@")[0]) for name, r in k.items())
    assert bench.measured_traffic("recur", "unit") == pytest.approx(11 * m)
    assert bench.measured_traffic("recur", "other") is None


def test_ingest_needs_the_copy(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "traffic.json"))
    _counter_csv(tmp_path / "f.csv", "FETCH_SIZE", [("kda::prep_kernel()", 1.0)])
    _counter_csv(tmp_path / "w.csv", "WRITE_SIZE", [("kda::prep_kernel()", 1.0)])
    with pytest.raises(SystemExit):
        bench.ingest_pmc(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"), "unit", "cmd")
