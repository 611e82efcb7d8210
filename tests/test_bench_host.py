"""Host logic of bench.py, on the CPU: the one-GPU contract and the
arithmetic that turns rocprofv3 counter readings into the bytes per call
that the bench line reports as its roofline's traffic."""
import csv
import json
import os
import subprocess
import sys

import pytest

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = "void kda::prefill_wy_prep_kernel<0, false>(unsigned short const*, float const*)"
OTHER = "void at::native::vectorized_elementwise_kernel<4, fill>(int)"
COPY = "__amd_rocclr_copyBuffer"


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_kernel_short_names():
    assert bench.kernel_short(LIB) == "prefill_wy_prep_kernel<0, false>"
    assert bench.kernel_short(OTHER) is None
    assert bench.kernel_short(COPY) is None


def _write(path, header, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(header)
        w.writerows(rows)


def test_digest_counters_arithmetic(tmp_path, monkeypatch):
    # one library dispatch per counter workload, separated by a foreign
    # kernel, then the calibration copy: FETCH_SIZE reads half the copy's
    # bytes (factor 2), WRITE_SIZE all of them (factor 1)
    nw = len(bench.COUNTER_WORKLOADS)
    names = []
    for i in range(nw):
        names += [LIB, OTHER]
    names[-1] = COPY
    copy_kib = bench.COPY_BYTES / 1024.0
    trace, fetch, write, mfma = [], [], [], []
    for d, n in enumerate(names):
        trace.append([d, n, 1000 * d, 1000 * d + (5000 if n == LIB else 100)])
        fetch.append([d, n, 100.0 if n == LIB else (copy_kib / 2 if n == COPY else 7.0)])
        write.append([d, n, 50.0 if n == LIB else (copy_kib if n == COPY else 7.0)])
        mfma.append([d, n, 10.0 if n == LIB else 0.0])
    folder = tmp_path / "out"
    _write(str(folder / "ks" / "ks_kernel_trace.csv"),
           ["Dispatch_Id", "Kernel_Name", "Start_Timestamp", "End_Timestamp"], trace)
    for c, rows in (("FETCH_SIZE", fetch), ("WRITE_SIZE", write), ("MfmaUtil", mfma)):
        _write(str(folder / ("pmc_" + c) / "pmc_counter_collection.csv"),
               ["Dispatch_Id", "Kernel_Name", "Counter_Value"], rows)
    (tmp_path / "profiles").mkdir()
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "source_digest", lambda: "digest-under-test")
    bench.digest_counters(str(folder))

    rec = json.load(open(tmp_path / "profiles" / "traffic.json"))
    assert rec["source_digest"] == "digest-under-test"
    assert rec["calibration"]["fetch_factor"] == pytest.approx(2.0)
    assert rec["calibration"]["write_factor"] == pytest.approx(1.0)
    per_dispatch = 100 * 1024 * 2.0 + 50 * 1024 * 1.0
    for wname, scale in bench.COUNTER_WORKLOADS:
        w = rec["workloads"][wname]
        k = w["kernels"]["prefill_wy_prep_kernel<0, false>"]
        assert k["dispatches"] == 1
        assert k["read_bytes"] == pytest.approx(100 * 1024 * 2.0)
        assert k["written_bytes"] == pytest.approx(50 * 1024.0)
        assert k["avg_us"] == pytest.approx(5.0)
        assert k["mfma_busy_pct"] == pytest.approx(10.0)
        assert w["measured_bytes"] == pytest.approx(per_dispatch)
        assert w["bytes_per_call"] == pytest.approx(per_dispatch * scale)
        assert w["us_per_call"] == pytest.approx(5.0 * scale)
    md = open(tmp_path / "profiles" / bench.COUNTERS_MD).read()
    assert "digest-under-test" in md and "long_t1m_prefill" in md


def test_committed_traffic_record_shape():
    # the committed record names every counter workload and its calibration
    rec = json.load(open(os.path.join(ROOT, "profiles", "traffic.json")))
    assert set(rec["workloads"]) == {w for w, _ in bench.COUNTER_WORKLOADS}
    assert rec["calibration"]["fetch_factor"] > 0 and rec["calibration"]["write_factor"] > 0
    for w in rec["workloads"].values():
        assert w["bytes_per_call"] > 0 and w["us_per_call"] > 0
