"""Host-side logic of bench.py: the refusal of several GPUs and the parsers of rocprofv3 CSV output.

No GPU is touched: the CSVs are tiny synthetic files in the layout rocprofv3 writes (kernel trace:
Kernel_Name, Start_Timestamp, End_Timestamp in ns; counter collection: Dispatch_Id, Kernel_Name,
Counter_Name, Counter_Value with one row per counter instance).
"""
import csv
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

import bench  # noqa: E402


def write_csv(path, header, rows):
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(header)
        w.writerows(rows)
    return str(path)


@pytest.mark.parametrize("n", [0, 2, 8])
def test_several_gpus_refused(n):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", str(n)],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "measures one GPU" in r.stderr and f"--gpus {n}" in r.stderr
    assert r.stdout == ""


def test_short_kernel_names():
    assert bench.short_kernel("diff_band(unsigned int, float const*) [clone .kd]") == "diff_band"
    assert bench.short_kernel("void attn_bf16_quad<true>(Args)") == "attn_bf16_quad"
    assert bench.short_kernel("__amd_rocclr_copyBuffer.kd") == bench.COPY_KERNEL
    assert bench.short_kernel("some_other_kernel") == "some_other_kernel"


def test_trace_summary(tmp_path):
    rows = [("attn_bf16_quad", 1000, 1000 + d) for d in (80_000, 84_000, 90_000)]
    rows += [("xattn_bf16", 5, 5 + 6_500)]
    p = write_csv(tmp_path / "kt.csv", ["Kernel_Name", "Start_Timestamp", "End_Timestamp"], rows)
    out = bench.trace_summary(p)
    # sorted by total time, largest first
    assert [r["kernel"] for r in out] == ["attn_bf16_quad", "xattn_bf16"]
    a = out[0]
    assert a["launches"] == 3
    assert a["median_us"] == 84.0 and a["min_us"] == 80.0 and a["max_us"] == 90.0
    assert a["mean_us"] == pytest.approx((80 + 84 + 90) / 3, abs=1e-3)
    assert out[1] == {"kernel": "xattn_bf16", "launches": 1, "median_us": 6.5, "mean_us": 6.5,
                      "min_us": 6.5, "max_us": 6.5}


COUNTER_HEADER = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]


def test_counter_means_sums_instances(tmp_path):
    # two dispatches of one kernel, each counter reported per instance (summed within a dispatch)
    rows = [(1, "diff_band.kd", "SQ_WAVES", 10), (1, "diff_band.kd", "SQ_WAVES", 30),
            (2, "diff_band.kd", "SQ_WAVES", 20), (2, "diff_band.kd", "SQ_WAVES", 20),
            (3, "xattn_bf16.kd", "SQ_WAVES", 7)]
    p = write_csv(tmp_path / "c.csv", COUNTER_HEADER, rows)
    vals = bench.counter_values(p)
    assert vals["diff_band"]["SQ_WAVES"] == {"1": 40.0, "2": 40.0}
    means, n = bench.counter_means(p)
    assert means == {"diff_band": {"SQ_WAVES": 40.0}, "xattn_bf16": {"SQ_WAVES": 7.0}}
    assert n == {"diff_band": 2, "xattn_bf16": 1}


def test_traffic_summary_scales_by_copy(tmp_path):
    copy_kib = (256 << 20) // 1024
    # the counters read 1.25x (fetch) and 0.8x (write) of the true bytes on the copy; the calibration copy
    # is the largest copy dispatch, a small upload runs the same kernel earlier
    fetch = [(1, bench.COPY_KERNEL, "FETCH_SIZE", 64), (2, bench.COPY_KERNEL, "FETCH_SIZE", 1.25 * copy_kib),
             (3, "diff_band.kd", "FETCH_SIZE", 1000.0), (4, "diff_band.kd", "FETCH_SIZE", 1500.0)]
    write = [(1, bench.COPY_KERNEL, "WRITE_SIZE", 64), (2, bench.COPY_KERNEL, "WRITE_SIZE", 0.8 * copy_kib),
             (3, "diff_band.kd", "WRITE_SIZE", 400.0), (4, "diff_band.kd", "WRITE_SIZE", 400.0)]
    pf = write_csv(tmp_path / "f.csv", COUNTER_HEADER, fetch)
    pw = write_csv(tmp_path / "w.csv", COUNTER_HEADER, write)
    out = bench.traffic_summary(pf, pw)
    assert out["fetch_scale"] == pytest.approx(1 / 1.25)
    assert out["write_scale"] == pytest.approx(1 / 0.8)
    b = out["diff_band"]
    assert b["dispatches"] == [2, 2]
    assert b["fetch_kib"] == 1250.0 and b["write_kib"] == 400.0
    assert b["hbm_bytes_per_launch"] == round(1250 * 1024 / 1.25 + 400 * 1024 / 0.8)
    assert b["source_digest"] == bench.source_digest(bench.KERNEL_SOURCES["diff_band"])
    # kernels seen in only one of the two runs are left out
    assert "xattn_bf16" not in out


def test_traffic_for_checks_digest(tmp_path, monkeypatch):
    src = bench.KERNEL_SOURCES["diff_band"]
    good = {"sources": src, "source_digest": bench.source_digest(src), "hbm_bytes_per_launch": 123}
    stale = dict(good, source_digest="0" * 16)
    p = tmp_path / "traffic.json"
    p.write_text(json.dumps({"diff_band": good, "xattn_bf16": stale}))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(p))
    assert bench.traffic_for("diff_band") == 123
    assert bench.traffic_for("xattn_bf16") is None      # source changed since the counters were taken
    assert bench.traffic_for("attn_bf16_quad") is None  # never profiled
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "missing.json"))
    assert bench.traffic_for("diff_band") is None


def test_cli_summaries(tmp_path):
    p = write_csv(tmp_path / "kt.csv", ["Kernel_Name", "Start_Timestamp", "End_Timestamp"],
                  [("diff_band", 0, 38_700)])
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--trace-summary", p],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    assert json.loads(r.stdout.strip())["median_us"] == 38.7
