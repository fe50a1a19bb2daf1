"""Turn rocprofv3 CSV output into the short text summaries kept under profiles/.

Usage (from the repository root, after copying rocprofv3 output back):

    python -m fp8_fine_grained_amd.profile_summary stats <kernel_stats.csv> <out.md> "<command>" [bench.log]
    python -m fp8_fine_grained_amd.profile_summary traffic <fetch.csv> <write.csv> \
        <calib_fetch.csv> <calib_write.csv> <kernel-substring> <kernel-source> <out.md> \
        "<fetch command>" "<write command>" "<calibration commands>"
    python -m fp8_fine_grained_amd.profile_summary mfma <counters.csv> <kernel-substring> <last-n> \
        <kernel-source> <out.md> "<command>"

``mfma`` reads one counter pass (SQ_VALU_MFMA_BUSY_CYCLES, GRBM_GUI_ACTIVE (summed
over the 8 XCDs, so divided by 8 for one XCD's active cycles),
SQ_INSTS_VALU_MFMA_MOPS_F8 / _F16, SQ_BUSY_CYCLES, LDS counters) over the kernel's
last n dispatches and derives the matrix-core utilisation (MFMA-busy SIMD
cycles over active cycles times the 1024 SIMDs), the average clock (active
cycles over the dispatch's duration) and the matrix-core flop rate.

``traffic`` averages the FETCH_SIZE / WRITE_SIZE counters (KiB per dispatch)
over the dispatches whose name contains the substring, and scales each by what
the same counter reads for a plain device-to-device copy of 1 GiB (the largest
dispatch of the calibration run): bytes = counter * 1024 * (known / measured).
The summary records the sha256 of the kernel source it was measured with;
``bench.py`` only reports the traffic while that source is unchanged.
"""

import csv
import hashlib
import os
import json
import sys

COPY_BYTES = 1 << 30


def _rows(path):
    with open(path) as f:
        return list(csv.DictReader(f))


def _bench_line(log_path):
    """The JSON line bench.py printed in the profiled run (None if absent)."""
    try:
        lines = open(log_path).read().splitlines()
    except OSError:
        return None
    for line in reversed(lines):
        if line.startswith("{") and '"metric"' in line:
            return json.loads(line)
    return None


def stats(csv_path, out_md, command, bench_log=None):
    rows = _rows(csv_path)
    lines = [
        "# rocprofv3 kernel statistics",
        "",
        "Command (run from the repository root):",
        "",
        "```",
        command,
        "```",
        "",
        "| kernel | calls | average (us) | min (us) | max (us) | share |",
        "|---|---|---|---|---|---|",
    ]
    for r in rows:
        name = r["Name"]
        if len(name) > 110:
            name = name[:107] + "..."
        lines.append(
            f"| `{name}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
            f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | {float(r['Percentage']):.1f}% |")
    bench = _bench_line(bench_log) if bench_log else None
    trace = os.path.join(os.path.dirname(csv_path), os.path.basename(csv_path).replace("kernel_stats", "kernel_trace"))
    if bench and os.path.exists(trace):
        # The timed launches are the last `steps` dispatches of each kernel and
        # launch shape (grid size): the bench's extra lines after the step (the
        # same quantisers on other shapes) have grids of their own.
        n = int(bench["steps"])
        durs = {}
        for r in _rows(trace):
            durs.setdefault((r["Kernel_Name"], int(r["Grid_Size_X"])), []).append(
                (int(r["Start_Timestamp"]), int(r["End_Timestamp"]) - int(r["Start_Timestamp"])))
        lines += ["", f"rocprofv3 average over the last {n} dispatches of each kernel and grid size (the timed",
                  "steps, and the last launches of each extra line):", "",
                  "| kernel | grid (threads) | dispatches | average (us) |", "|---|---|---|---|"]
        for (name, grid), d in durs.items():
            d = [x for _, x in sorted(d)][-n:]
            short = name if len(name) <= 110 else name[:107] + "..."
            lines.append(f"| `{short}` | {grid} | {len(d)} | {sum(d) / len(d) / 1e3:.2f} |")
    if bench:
        lines += ["", "bench.py's own HIP-event averages over the same timed steps (the first table also",
                  "counts the warm-up launches):", "", "| launch | ms |", "|---|---|"]
        for name, k in bench.get("kernels", {}).items():
            ms = k["ms"] if "ms" in k else (k["us"] / 1e3 if "us" in k else None)
            if ms is not None:
                lines.append(f"| {name} | {ms:.4f} |")
        lines.append(f"| whole step | {bench['ms_per_step']:.4f} |")
    with open(out_md, "w") as f:
        f.write("\n".join(lines) + "\n")


def _mean_counter(path, counter, substr=None, largest=False):
    vals = []
    for r in _rows(path):
        if r["Counter_Name"] != counter:
            continue
        if substr is not None and substr not in r["Kernel_Name"]:
            continue
        vals.append((float(r["Counter_Value"]), r["Kernel_Name"]))
    if not vals:
        raise SystemExit(f"no {counter} rows matching {substr!r} in {path}")
    if largest:
        v = max(vals)
        return v[0], v[1], 1
    return sum(v for v, _ in vals) / len(vals), vals[0][1], len(vals)


def traffic(fetch_csv, write_csv, cal_fetch_csv, cal_write_csv, substr, kernel_src, out_md,
            fetch_cmd, write_cmd, cal_cmd):
    f_kib, name, nf = _mean_counter(fetch_csv, "FETCH_SIZE", substr)
    w_kib, _, nw = _mean_counter(write_csv, "WRITE_SIZE", substr)
    cf_kib, cname, _ = _mean_counter(cal_fetch_csv, "FETCH_SIZE", largest=True)
    cw_kib, _, _ = _mean_counter(cal_write_csv, "WRITE_SIZE", largest=True)
    f_scale = COPY_BYTES / (cf_kib * 1024.0)
    w_scale = COPY_BYTES / (cw_kib * 1024.0)
    fetch_bytes = f_kib * 1024.0 * f_scale
    write_bytes = w_kib * 1024.0 * w_scale
    with open(kernel_src, "rb") as fh:
        sha = hashlib.sha256(fh.read()).hexdigest()
    rec = {
        "kernel": name[:200],
        "kernel_source": kernel_src,
        "kernel_source_sha256": sha,
        "dispatches_averaged": {"fetch": nf, "write": nw},
        "fetch_kib_raw": f_kib,
        "write_kib_raw": w_kib,
        "copy_calibration": {"bytes": COPY_BYTES, "kernel": cname[:120], "fetch_kib": cf_kib,
                             "write_kib": cw_kib, "fetch_scale": f_scale, "write_scale": w_scale},
        "fetch_bytes": fetch_bytes,
        "write_bytes": write_bytes,
        "per_launch_bytes": fetch_bytes + write_bytes,
    }
    lines = [
        "# HBM traffic per launch (rocprofv3 FETCH_SIZE / WRITE_SIZE, copy-calibrated)",
        "",
        f"Kernel: `{name[:160]}`",
        "",
        "Commands (run from the repository root, one counter per run):",
        "",
        "```",
        fetch_cmd,
        write_cmd,
        cal_cmd,
        "```",
        "",
        f"- FETCH_SIZE {f_kib:.0f} KiB/dispatch x {f_scale:.4f} = {fetch_bytes / 1e6:.1f} MB",
        f"- WRITE_SIZE {w_kib:.0f} KiB/dispatch x {w_scale:.4f} = {write_bytes / 1e6:.1f} MB",
        f"- calibration: 1 GiB copy read {cf_kib:.0f} KiB, wrote {cw_kib:.0f} KiB",
        "",
        "```json",
        json.dumps(rec, indent=1),
        "```",
    ]
    with open(out_md, "w") as f:
        f.write("\n".join(lines) + "\n")


SIMDS = 1024        # 256 CUs x 4 SIMDs
XCDS = 8            # GRBM_GUI_ACTIVE is reported summed over the 8 XCDs (one instance each)
PEAK_CLOCK_GHZ = 2.4


def mfma(csv_path, substr, last_n, kernel_src, out_md, command):
    last_n = int(last_n)
    per = {}  # dispatch -> {counter: value}, plus timestamps
    name = None
    for r in _rows(csv_path):
        if substr not in r["Kernel_Name"]:
            continue
        name = r["Kernel_Name"]
        d = per.setdefault(int(r["Dispatch_Id"]), {"_t": int(r["End_Timestamp"]) - int(r["Start_Timestamp"])})
        d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    if not per:
        raise SystemExit(f"no dispatches matching {substr!r} in {csv_path}")
    ds = [per[k] for k in sorted(per)][-last_n:]
    avg = {k: sum(d.get(k, 0.0) for d in ds) / len(ds) for k in ds[0]}
    t_s = avg["_t"] * 1e-9
    active = avg["GRBM_GUI_ACTIVE"] / XCDS  # cycles of one XCD (all run the whole dispatch)
    util = avg["SQ_VALU_MFMA_BUSY_CYCLES"] / (active * SIMDS)
    clock = active / t_s / 1e9
    flops8 = avg.get("SQ_INSTS_VALU_MFMA_MOPS_F8", 0.0) * 512
    flops16 = avg.get("SQ_INSTS_VALU_MFMA_MOPS_F16", 0.0) * 512
    lines = [
        "# Matrix-core utilisation (rocprofv3 counters)",
        "",
        f"Kernel: `{name[:160]}`",
        "",
        "Command (run from the repository root):",
        "",
        "```",
        command,
        "```",
        "",
        f"Averages over the kernel's last {len(ds)} dispatches (counters summed over all XCDs and shader engines):",
        "",
        "| quantity | value |",
        "|---|---|",
        f"| dispatch duration (counter run) | {t_s * 1e6:.1f} us |",
    ]
    for k in sorted(avg):
        if k != "_t":
            lines.append(f"| {k} | {avg[k]:.4g} |")
    lines += [
        f"| MFMA utilisation = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / {XCDS} XCDs x {SIMDS} SIMDs) | {util:.3f} |",
        f"| average clock = (GRBM_GUI_ACTIVE / {XCDS}) / duration | {clock:.2f} GHz |",
        f"| utilisation x clock / {PEAK_CLOCK_GHZ} GHz (fraction of the published peak's matrix-core cycles) | "
        f"{util * clock / PEAK_CLOCK_GHZ:.3f} |",
    ]
    if "SQ_WAVE_CYCLES" in avg:
        wc = avg["SQ_WAVE_CYCLES"]
        for k in ("SQ_WAIT_ANY", "SQ_WAIT_INST_ANY", "SQ_ACTIVE_INST_ANY", "SQ_ACTIVE_INST_VALU",
                  "SQ_ACTIVE_INST_LDS", "SQ_ACTIVE_INST_VMEM"):
            if k in avg:
                lines.append(f"| {k} / SQ_WAVE_CYCLES | {avg[k] / wc:.3f} |")
        lines.append(f"| resident wavefronts per SIMD = 4 x SQ_WAVE_CYCLES / (active cycles x {SIMDS}) | "
                     f"{4 * wc / (active * SIMDS):.2f} |")
    if avg.get("SQ_INSTS_MFMA"):
        if "SQ_INSTS_VALU" in avg:
            lines.append(f"| VALU instructions per MFMA = SQ_INSTS_VALU / SQ_INSTS_MFMA | "
                         f"{avg['SQ_INSTS_VALU'] / avg['SQ_INSTS_MFMA']:.2f} |")
    if avg.get("SQ_VALU_MFMA_BUSY_CYCLES") and "SQ_VALU_MFMA_COEXEC_CYCLES" in avg:
        lines.append(f"| VALU co-execution = SQ_VALU_MFMA_COEXEC_CYCLES / SQ_VALU_MFMA_BUSY_CYCLES | "
                     f"{avg['SQ_VALU_MFMA_COEXEC_CYCLES'] / avg['SQ_VALU_MFMA_BUSY_CYCLES']:.3f} |")
    if flops8:
        lines.append(f"| FP8 matrix-core work = MOPS_F8 x 512 | {flops8 / 1e9:.1f} GFLOP, {flops8 / t_s / 1e12:.0f} TFLOP/s |")
    if flops16:
        lines.append(f"| F16 matrix-core work = MOPS_F16 x 512 | {flops16 / 1e9:.1f} GFLOP, {flops16 / t_s / 1e12:.0f} TFLOP/s |")
    with open(kernel_src, "rb") as fh:
        sha = hashlib.sha256(fh.read()).hexdigest()
    rec = {"kernel": name[:200], "kernel_source": kernel_src, "kernel_source_sha256": sha,
           "dispatches_averaged": len(ds), "duration_us": t_s * 1e6, "mfma_busy_fraction": util,
           "clock_ghz": clock, "fraction_of_peak_mfma_cycles": util * clock / PEAK_CLOCK_GHZ}
    lines += ["", "```json", json.dumps(rec, indent=1), "```"]
    with open(out_md, "w") as f:
        f.write("\n".join(lines) + "\n")


def load_traffic(md_path):
    """The JSON record embedded in a traffic summary (None if absent)."""
    try:
        text = open(md_path).read()
    except OSError:
        return None
    start = text.find("```json")
    if start < 0:
        return None
    end = text.find("```", start + 7)
    try:
        return json.loads(text[start + 7:end])
    except ValueError:
        return None


if __name__ == "__main__":
    if sys.argv[1] == "stats":
        stats(*sys.argv[2:6])
    elif sys.argv[1] == "traffic":
        traffic(*sys.argv[2:12])
    elif sys.argv[1] == "mfma":
        mfma(*sys.argv[2:8])
    else:
        raise SystemExit(__doc__)
