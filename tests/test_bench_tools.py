"""Host-side logic of the benchmark and of the profile summaries (no GPU).

bench.py must refuse more than one GPU before touching the device; its
kernel-source hash must ignore comments and whitespace but not code; the
committed traffic figure is reported only for the source it was measured on.
bench_profile.py's summaries are checked on small synthetic rocprofv3 CSVs
whose expected figures follow by hand.
"""

import csv
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import bench_profile  # noqa: E402


def _write_csv(path, header, rows):
    with open(path, "w", newline="") as fh:
        w = csv.writer(fh)
        w.writerow(header)
        w.writerows(rows)
    return str(path)


def test_bench_refuses_more_than_one_gpu():
    proc = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                          capture_output=True, text=True, timeout=120)
    assert proc.returncode == 2
    assert "one GPU" in proc.stderr
    assert proc.stdout == ""


def test_source_hash_ignores_comments_not_code(tmp_path, monkeypatch):
    src = tmp_path / "k.hpp"
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "GEMM_SOURCES", ["k.hpp"])
    src.write_text("int f(int x) {\n  return x + 1;  // one more\n}\n")
    h0 = bench.gemm_source_hash()
    src.write_text("/* the successor */\nint f(int x)   {\n\n  return x + 1;  // plus one\n}\n")
    assert bench.gemm_source_hash() == h0
    src.write_text("int f(int x) {\n  return x + 2;\n}\n")
    assert bench.gemm_source_hash() != h0


def test_traffic_reported_only_for_its_source(tmp_path, monkeypatch):
    summary = tmp_path / "traffic.txt"
    summary.write_text("# L2-miss traffic\nsource_hash = abc123\nl2_miss_bytes_per_launch = 1880992992\n")
    monkeypatch.setattr(bench, "TRAFFIC_SUMMARY", str(summary))
    assert bench.read_traffic("abc123") == 1880992992.0
    assert bench.read_traffic("def456") is None
    monkeypatch.setattr(bench, "TRAFFIC_SUMMARY", str(tmp_path / "missing.txt"))
    assert bench.read_traffic("abc123") is None


TRACE_HEADER = ["Kernel_Name", "Start_Timestamp", "End_Timestamp", "Workgroup_Size_X", "Workgroup_Size_Y",
                "Workgroup_Size_Z", "Grid_Size_X", "Grid_Size_Y", "Grid_Size_Z"]


def test_stats_by_grid_keeps_shapes_apart(tmp_path):
    # one kernel at 1024 and 256 workgroups of 256 threads, another kernel once
    rows = [["gemm<A>", 0, 700_000, 256, 1, 1, 1024 * 256, 1, 1],
            ["gemm<A>", 0, 720_000, 256, 1, 1, 1024 * 256, 1, 1],
            ["gemm<A>", 0, 180_000, 256, 1, 1, 256 * 256, 1, 1],
            ["copy", 10, 50_010, 512, 1, 1, 4096 * 512, 1, 1]]
    path = _write_csv(tmp_path / "trace.csv", TRACE_HEADER, rows)
    got = {(k["name"], k["workgroups"]): k for k in bench_profile.kernel_stats_by_grid(path)}
    assert set(got) == {("gemm<A>", 1024), ("gemm<A>", 256), ("copy", 4096)}
    big = got[("gemm<A>", 1024)]
    assert big["calls"] == 2 and big["avg_ns"] == 710_000 and big["min_ns"] == 700_000 and big["max_ns"] == 720_000
    assert got[("gemm<A>", 256)]["avg_ns"] == 180_000
    assert got[("copy", 4096)]["avg_ns"] == 50_000
    only = bench_profile.kernel_stats_by_grid(path, match="copy")
    assert [k["name"] for k in only] == ["copy"]


COUNTER_HEADER = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value", "Start_Timestamp",
                  "End_Timestamp"]


def test_traffic_calibrated_by_the_copy(tmp_path):
    # FETCH_SIZE reads a 1 GiB copy as 512 MiB (scale 2), WRITE_SIZE exactly; the
    # kernel's values are split over two counter instances per dispatch
    gib_kib = (1 << 30) / 1024
    fetch = _write_csv(tmp_path / "fetch.csv", COUNTER_HEADER, [
        [1, "gemm<A>", "FETCH_SIZE", 300_000, 0, 1], [1, "gemm<A>", "FETCH_SIZE", 100_000, 0, 1],
        [2, "gemm<A>", "FETCH_SIZE", 400_000, 0, 1],
        [3, "__amd_rocclr_copyBuffer", "FETCH_SIZE", gib_kib / 2, 0, 1]])
    write = _write_csv(tmp_path / "write.csv", COUNTER_HEADER, [
        [1, "gemm<A>", "WRITE_SIZE", 262_144, 0, 1], [2, "gemm<A>", "WRITE_SIZE", 262_144, 0, 1],
        [3, "__amd_rocclr_copyBuffer", "WRITE_SIZE", gib_kib, 0, 1]])
    t = bench_profile.traffic(fetch, write, "gemm<A>")
    assert t["fetch_scale"] == pytest.approx(2.0) and t["write_scale"] == pytest.approx(1.0)
    assert t["fetch_bytes"] == pytest.approx(400_000 * 1024 * 2.0)
    assert t["write_bytes"] == pytest.approx(262_144 * 1024)
    assert t["l2_miss_bytes_per_launch"] == pytest.approx(400_000 * 2048 + 262_144 * 1024)
    assert t["dispatches"] == (2, 2)


def test_counters_derive_clock_and_busy(tmp_path):
    # one XCD active for 1.8e6 cycles over 1 ms: 1.8 GHz; busy 80% of 1024 SIMDs x those cycles
    cycles, dur_ns = 1.8e6, 1_000_000
    busy = 0.8 * 1024 * cycles
    rows = []
    for d in (1, 2, 3):        # the first dispatch is dropped (skip = 1)
        scale = 0.5 if d == 1 else 1.0
        rows += [[d, "gemm<A>", "MfmaUtil", 80.0, 0, dur_ns],
                 [d, "gemm<A>", "SQ_VALU_MFMA_BUSY_CYCLES", busy * scale, 0, dur_ns],
                 [d, "gemm<A>", "SQ_LDS_BANK_CONFLICT", 10.0, 0, dur_ns],
                 [d, "gemm<A>", "SQ_LDS_IDX_ACTIVE", 1000.0, 0, dur_ns]]
    path = _write_csv(tmp_path / "pmc.csv", COUNTER_HEADER, rows)
    out, derived = bench_profile.counters([path], "gemm<A>", skip=1, trace_us=900.0)
    assert out["SQ_VALU_MFMA_BUSY_CYCLES"] == pytest.approx(busy)
    assert derived["mfma_busy_pct"] == pytest.approx(80.0)
    assert derived["clock_ghz_under_counters"] == pytest.approx(1.8)
    assert derived["active_cycles_per_xcd"] == pytest.approx(cycles)
    assert derived["clock_ghz_at_trace_duration"] == pytest.approx(cycles / 900e3)
    assert derived["lds_conflict_cycles_per_active_cycle"] == pytest.approx(0.01)
    assert derived["dispatches_used_per_pass"] == 2


def test_traffic_summary_reports_the_expected_fetch(tmp_path):
    gib_kib = (1 << 30) / 1024
    fetch = _write_csv(tmp_path / "fetch.csv", COUNTER_HEADER, [
        [1, "gemm<A>", "FETCH_SIZE", 500_000, 0, 1], [2, "__amd_rocclr_copyBuffer", "FETCH_SIZE", gib_kib / 2, 0, 1]])
    write = _write_csv(tmp_path / "write.csv", COUNTER_HEADER, [
        [1, "gemm<A>", "WRITE_SIZE", 1000, 0, 1], [2, "__amd_rocclr_copyBuffer", "WRITE_SIZE", gib_kib, 0, 1]])
    out = tmp_path / "t.txt"
    bench_profile.main(["traffic", "--fetch", fetch, "--write", write, "--match", "gemm<A>",
                        "--algorithmic-bytes", "1e9", "--expected-fetch-bytes", str(500_000 * 2048),
                        "--expected-note", "by hand", "--source-hash", "h", "--command", "c", "--out", str(out)])
    kv = dict(line.split(" = ", 1) for line in out.read_text().splitlines() if " = " in line and line[0] != "#")
    assert float(kv["fetch_over_expected"]) == pytest.approx(1.0)
    assert float(kv["expected_fetch_bytes"]) == 500_000 * 2048
    assert kv["source_hash"] == "h"
