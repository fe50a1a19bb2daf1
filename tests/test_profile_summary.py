"""CPU checks of the measurement evidence pipeline: the rocprofv3 CSV summaries
(copy-calibrated traffic, matrix-core utilisation and clock) computed from
synthetic counter files with known answers, and bench.py reporting a summary's
figures only while the kernel source it was taken on is unchanged."""

import csv
import hashlib
import math
import os

import bench
from fp8_fine_grained_amd import profile_summary as ps

FIELDS = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value", "Start_Timestamp", "End_Timestamp"]


def _write(path, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=FIELDS)
        w.writeheader()
        for r in rows:
            w.writerow(r)


def _row(d, name, counter, value, t0=0, t1=1_000_000):
    return {"Dispatch_Id": d, "Kernel_Name": name, "Counter_Name": counter, "Counter_Value": value,
            "Start_Timestamp": t0, "End_Timestamp": t1}


def test_traffic_is_copy_calibrated(tmp_path):
    src = tmp_path / "k.hip"
    src.write_text("kernel source\n")
    fetch, write = tmp_path / "f.csv", tmp_path / "w.csv"
    cf, cw = tmp_path / "cf.csv", tmp_path / "cw.csv"
    # two dispatches of the kernel (1000 and 1200 KiB fetched), one of another
    _write(fetch, [_row(1, "gemm_x", "FETCH_SIZE", 1000), _row(2, "gemm_x", "FETCH_SIZE", 1200),
                   _row(3, "other", "FETCH_SIZE", 99999)])
    _write(write, [_row(1, "gemm_x", "WRITE_SIZE", 500), _row(2, "gemm_x", "WRITE_SIZE", 500)])
    # the 1 GiB copy reads 512 Ki KiB (half of 1 GiB: the counter sees half) and writes 1 Gi
    _write(cf, [_row(1, "copy", "FETCH_SIZE", 524288), _row(2, "small", "FETCH_SIZE", 10)])
    _write(cw, [_row(1, "copy", "WRITE_SIZE", 1048576)])
    out = tmp_path / "t.md"
    ps.traffic(str(fetch), str(write), str(cf), str(cw), "gemm_x", str(src), str(out), "f", "w", "c")
    rec = ps.load_traffic(str(out))
    assert rec["copy_calibration"]["fetch_scale"] == 2.0 and rec["copy_calibration"]["write_scale"] == 1.0
    assert rec["fetch_bytes"] == 1100 * 1024 * 2.0
    assert rec["write_bytes"] == 500 * 1024
    assert rec["per_launch_bytes"] == rec["fetch_bytes"] + rec["write_bytes"]
    assert rec["kernel_source_sha256"] == hashlib.sha256(b"kernel source\n").hexdigest()


def test_mfma_utilisation_and_clock(tmp_path):
    src = tmp_path / "k.hip"
    src.write_text("x")
    rows = []
    # three dispatches of 1 ms; the last two at 2.0 GHz with the matrix cores busy half the time
    for d, (ghz, busy) in enumerate([(1.0, 0.9), (2.0, 0.5), (2.0, 0.5)], start=1):
        active = ghz * 1e9 * 1e-3  # cycles of one XCD over 1 ms
        rows += [_row(d, "gemm_y", "GRBM_GUI_ACTIVE", 8 * active),
                 _row(d, "gemm_y", "SQ_VALU_MFMA_BUSY_CYCLES", busy * active * 1024),
                 _row(d, "gemm_y", "SQ_INSTS_VALU_MFMA_MOPS_F8", 1e6)]
    csv_path = tmp_path / "m.csv"
    _write(csv_path, rows)
    out = tmp_path / "m.md"
    ps.mfma(str(csv_path), "gemm_y", 2, str(src), str(out), "cmd")
    rec = ps.load_traffic(str(out))
    assert rec["dispatches_averaged"] == 2
    assert math.isclose(rec["clock_ghz"], 2.0) and math.isclose(rec["mfma_busy_fraction"], 0.5)
    assert math.isclose(rec["fraction_of_peak_mfma_cycles"], 0.5 * 2.0 / 2.4)
    assert math.isclose(rec["duration_us"], 1000.0)
    text = out.read_text()
    assert "512.0 GFLOP" not in text and "0.5 GFLOP" in text  # 1e6 MOPS x 512 flops


def test_bench_reports_a_summary_only_for_its_source(tmp_path, monkeypatch):
    prof = tmp_path / "profiles"
    prof.mkdir()
    src_dir = tmp_path / "fp8_fine_grained_amd" / "csrc"
    src_dir.mkdir(parents=True)
    gemm = src_dir / "gemm_fp8.hip"
    gemm.write_text("version 1\n")
    rows = []
    for d in (1, 2):
        rows += [_row(d, "gemm_z", "GRBM_GUI_ACTIVE", 8 * 2e6), _row(d, "gemm_z", "SQ_VALU_MFMA_BUSY_CYCLES", 1e9)]
    _write(tmp_path / "m.csv", rows)
    ps.mfma(str(tmp_path / "m.csv"), "gemm_z", 2, str(gemm), str(prof / "rec.md"), "cmd")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    got = bench._mfma_counters("rec.md")
    assert got is not None and math.isclose(got["clock_ghz"], 2.0)
    gemm.write_text("version 2\n")  # the kernel source changed since the counters were taken
    assert bench._mfma_counters("rec.md") is None
    assert bench._mfma_counters("missing.md") is None
