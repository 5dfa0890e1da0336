"""Text summaries of rocprofv3 CSV output for the kernels bench.py reports.

    python profsum.py trace   TRACE_DIR BENCH_OUT  "<command>"
    python profsum.py stats   TRACE_DIR -          "<command>"
    python profsum.py traffic FETCH_DIR WRITE_DIR  "<command>"
    python profsum.py pmc     PMC_DIR   KERNEL     "<command>"

``trace`` reads ``*_kernel_stats.csv`` and ``*_kernel_trace.csv`` of a ``--kernel-trace
--stats -f csv`` run of bench.py and prints the per-kernel table plus the average
duration of the dominant launch (the gate|up forward at the 8B shape, recognised by its
kernel name and grid) over the benchmark's timed launches, beside the benchmark's own
HIP-event average from the same run (BENCH_OUT: the file holding bench.py's JSON line).

``stats`` prints the per-kernel table of a kernel-trace run (every kernel, by total time).

``traffic`` reads the ``*_counter_collection.csv`` of two ``--pmc FETCH_SIZE`` and
``--pmc WRITE_SIZE`` runs and scales each counter by what it reads for the benchmark's
calibration kernel (a float32 elementwise copy of 256 MiB in, 256 MiB out), giving HBM
bytes per launch of the dominant kernel and of the NF4 input-gradient launch of the same
group.  The printed ``kernel_source_sha256`` ties the figures to the kernel sources they
were taken on.

``pmc`` prints, for every counter of a ``--kernel-trace --pmc`` run, its per-dispatch
average over the dominant launches (KERNEL "-") or over every launch whose name contains
KERNEL, plus the derived clock (one XCD's GUI-active cycles
over the dispatch's duration) and the MFMA-busy, LDS and wait fractions where the counters
for them are present.

The dominant kernel is named by ``bench.DOM_KERNEL`` / ``bench.DOM_GRID``; this script
sits beside bench.py and reads those definitions from it.
"""
from __future__ import annotations

import csv
import glob
import json
import os
import sys

sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
import bench  # noqa: E402  (the dominant kernel's name, grid and the kernel-source hash)

CAL_NAME = "neg_kernel"
CAL_BYTES = 256 << 20


def _one(pattern: str) -> str:
    hits = sorted(glob.glob(pattern, recursive=True))
    if not hits:
        raise SystemExit(f"no file matches {pattern}")
    return hits[0]


def _short(name: str, n: int = 70) -> str:
    return name if len(name) <= n else name[: n - 3] + "..."


def _bench_line(path: str):
    with open(path) as fh:
        for line in fh:
            line = line.strip()
            if line.startswith("{") and '"roofline"' in line:
                return json.loads(line)
    return None


def trace(trace_dir: str, bench_out: str, command: str) -> str:
    stats_rows = list(csv.DictReader(open(_one(os.path.join(trace_dir, "**", "*kernel_stats.csv")))))
    rows = list(csv.DictReader(open(_one(os.path.join(trace_dir, "**", "*kernel_trace.csv")))))
    b = _bench_line(bench_out)
    out = [f"# rocprofv3 kernel trace: {command}", ""]
    out.append(f"{'kernel':72s} {'calls':>6s} {'avg_us':>10s} {'min_us':>9s} {'max_us':>9s} {'share%':>7s}")
    for r in stats_rows[:20]:
        out.append(f"{_short(r['Name'], 72):72s} {int(r['Calls']):6d} {float(r['AverageNs']) / 1e3:10.2f} "
                   f"{float(r['MinNs']) / 1e3:9.2f} {float(r['MaxNs']) / 1e3:9.2f} {float(r['Percentage']):7.2f}")
    dom = sorted((int(r["Start_Timestamp"]), int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
                 for r in rows if bench.DOM_KERNEL in r["Kernel_Name"] and int(r["Grid_Size_X"]) == bench.DOM_GRID)
    out.append("")
    out.append(f"dominant launch: {bench.DOM_KERNEL} with grid {bench.DOM_GRID} (gate|up forward, M=2048 N=28672 K=4096)")
    out.append(f"  dispatches in the trace: {len(dom)}")
    if b is not None and dom:
        # the bench's warm-up steps come first, then its timed steps
        n = int(b["roofline"]["launches_timed"])
        skip = int(b["warmup"]) * (n // int(b["steps"]))
        timed = [d for _, d in dom[skip:skip + n]]
        avg = sum(timed) / len(timed) / 1e6
        out.append(f"  timed-region dispatches (#{skip}..#{skip + n - 1}): avg {avg:.4f} ms, "
                   f"min {min(timed) / 1e6:.4f} ms, max {max(timed) / 1e6:.4f} ms")
        out.append(f"  bench.py HIP-event average in the same run: {b['roofline']['avg_launch_ms']:.4f} ms "
                   f"(ratio {b['roofline']['avg_launch_ms'] / avg:.3f})")
        out.append(f"  achieved: {b['roofline']['flops_per_launch'] / (avg / 1e3) / 1e12:.1f} TFLOP/s from the "
                   f"trace average = {b['roofline']['flops_per_launch'] / (avg / 1e3) / 1e12 / bench.PEAK_BF16_TFLOPS:.4f}"
                   f" of {bench.PEAK_BF16_TFLOPS:.0f}")
        out.append(f"  bench.py ms_per_step {b['ms_per_step']}, value {b['value']} {b['unit']}")
    return "\n".join(out) + "\n"


def _rows(dir_: str):
    return list(csv.DictReader(open(_one(os.path.join(dir_, "**", "*counter_collection.csv")))))


def _avg(rows, counter: str, name: str, grid=None):
    vals = [float(r["Counter_Value"]) for r in rows
            if r["Counter_Name"] == counter and name in r["Kernel_Name"]
            and (grid is None or int(r["Grid_Size"]) == grid)]
    return (sum(vals) / len(vals), len(vals)) if vals else (None, 0)


def traffic(fetch_dir: str, write_dir: str, command: str) -> str:
    fr, wr = _rows(fetch_dir), _rows(write_dir)
    f_cal, _ = _avg(fr, "FETCH_SIZE", CAL_NAME)
    w_cal, _ = _avg(wr, "WRITE_SIZE", CAL_NAME)
    if f_cal is None or w_cal is None:
        raise SystemExit("calibration kernel missing")
    f_fac = f_cal * 1024.0 / CAL_BYTES
    w_fac = w_cal * 1024.0 / CAL_BYTES
    wl = bench.workload("llama8b")
    lines = [
        f"# HBM traffic per launch (gate|up group at the 8B shape, M=2048, N=28672 / K=28672)",
        f"# command: {command}",
        "# each counter is scaled by its reading for the calibration copy (256 MiB read, 256 MiB written)",
        f"kernel_source_sha256: {bench.kernel_source_hash()}",
        f"calibration_fetch_kib: {f_cal:.1f}",
        f"calibration_write_kib: {w_cal:.1f}",
        f"fetch_scale: {f_fac:.5f}",
        f"write_scale: {w_fac:.5f}",
    ]
    for tag, name, grid, alg in (("", bench.DOM_KERNEL, bench.DOM_GRID, bench.fwd_bytes(wl, ("gate", "up"))),
                                 ("dx_", bench.DX_KERNEL, bench.DX_GRID, bench.dx_bytes(wl, ("gate", "up")))):
        f_dom, f_n = _avg(fr, "FETCH_SIZE", name, grid)
        w_dom, w_n = _avg(wr, "WRITE_SIZE", name, grid)
        if f_dom is None or w_dom is None:
            lines.append(f"# {name} grid {grid}: not in this run")
            continue
        fetch_b = f_dom * 1024.0 / f_fac
        write_b = w_dom * 1024.0 / w_fac
        lines += [
            f"{tag}kernel: {name} grid {grid}",
            f"{tag}fetch_kib_per_launch: {f_dom:.1f}",
            f"{tag}fetch_launches: {f_n}",
            f"{tag}write_kib_per_launch: {w_dom:.1f}",
            f"{tag}write_launches: {w_n}",
            f"{tag}fetch_bytes_per_launch: {fetch_b:.0f}",
            f"{tag}write_bytes_per_launch: {write_b:.0f}",
            f"{tag}traffic_bytes_per_launch: {fetch_b + write_b:.0f}",
            f"{tag}algorithmic_bytes_per_launch: {alg}",
            f"{tag}traffic_over_algorithmic: {(fetch_b + write_b) / alg:.3f}",
        ]
    return "\n".join(lines) + "\n"


def pmc(pmc_dir: str, kernel: str, command: str) -> str:
    """Per-dispatch averages of every counter over the dominant launches (KERNEL "-"), or
    over every launch whose name contains KERNEL, and the derived clock and busy fractions.
    rocprofv3 sums a counter over its instances: GRBM_GUI_ACTIVE over the 8 XCDs (so one
    XCD's cycles are a 1/8 of it), SQ counters over every shader engine; the chip has 256
    compute units and 1024 SIMDs."""
    rows = _rows(pmc_dir)
    dom = kernel == "-"
    per = {}
    for r in rows:
        if (bench.DOM_KERNEL in r["Kernel_Name"] and int(r["Grid_Size"]) == bench.DOM_GRID) if dom else kernel in r["Kernel_Name"]:
            d = per.setdefault(r["Dispatch_Id"], {})
            d[r["Counter_Name"]] = float(r["Counter_Value"])
            d["dur_s"] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e9
    if not per:
        raise SystemExit("dominant kernel not in this run")
    names = sorted({k for d in per.values() for k in d})
    avg = {k: sum(d[k] for d in per.values() if k in d) / sum(1 for d in per.values() if k in d) for k in names}
    what = (f"{bench.DOM_KERNEL} grid {bench.DOM_GRID} (gate|up forward, M=2048 N=28672 K=4096)" if dom
            else f"every launch of {kernel}")
    out = [f"# rocprofv3 counters of {what}",
           f"# command: {command}",
           f"kernel_source_sha256: {bench.kernel_source_hash()}",
           f"dispatches: {len(per)}"]
    for k in names:
        out.append(f"{k}: {avg[k]:.6g}" if k != "dur_s" else f"duration_ms: {avg[k] * 1e3:.4f}")
    if "GRBM_GUI_ACTIVE" in avg:
        gui = avg["GRBM_GUI_ACTIVE"] / 8.0
        out.append(f"cycles_per_xcd: {gui:.0f}")
        out.append(f"clock_GHz (cycles / duration): {gui / avg['dur_s'] / 1e9:.3f}")
        if dom:
            flops = 2.0 * 2048 * 28672 * 4096
            out.append(f"achieved_TFLOPs: {flops / avg['dur_s'] / 1e12:.1f} ({flops / avg['dur_s'] / 1e12 / bench.PEAK_BF16_TFLOPS:.4f} of "
                       f"{bench.PEAK_BF16_TFLOPS:.0f}, a peak taken at 2.4 GHz)")
        derived = (("SQ_VALU_MFMA_BUSY_CYCLES", 1024, "mfma_busy_fraction (per SIMD)"),
                   ("SQ_LDS_IDX_ACTIVE", 256, "lds_active_fraction (per CU)"),
                   ("SQ_LDS_BANK_CONFLICT", 256, "lds_bank_conflict_fraction (per CU)"),
                   ("SQ_ACTIVE_INST_VALU", 1024, "valu_issue_fraction (per SIMD)"))
        for k, units, label in derived:
            if k in avg:
                out.append(f"{label}: {avg[k] / (gui * units):.4f}")
    if "SQ_WAVE_CYCLES" in avg:
        for k in ("SQ_WAIT_ANY", "SQ_WAIT_INST_ANY", "SQ_WAIT_INST_LDS"):
            if k in avg:
                out.append(f"{k} / SQ_WAVE_CYCLES: {avg[k] / avg['SQ_WAVE_CYCLES']:.4f}")
    if "SQ_INSTS_MFMA" in avg and dom:
        out.append(f"mfma_instructions: {avg['SQ_INSTS_MFMA']:.0f} (2 M N K / 32768 = {2.0 * 2048 * 28672 * 4096 / 32768:.0f})")
    return "\n".join(out) + "\n"


def stats(trace_dir: str, _unused: str, command: str) -> str:
    rows = list(csv.DictReader(open(_one(os.path.join(trace_dir, "**", "*kernel_stats.csv")))))
    out = [f"# rocprofv3 kernel statistics: {command}", ""]
    out.append(f"{'kernel':72s} {'calls':>6s} {'total_ms':>10s} {'avg_us':>10s} {'min_us':>9s} {'max_us':>9s} {'share%':>7s}")
    for r in rows:
        out.append(f"{_short(r['Name'], 72):72s} {int(r['Calls']):6d} {float(r['TotalDurationNs']) / 1e6:10.2f} "
                   f"{float(r['AverageNs']) / 1e3:10.2f} {float(r['MinNs']) / 1e3:9.2f} {float(r['MaxNs']) / 1e3:9.2f} "
                   f"{float(r['Percentage']):7.2f}")
    return "\n".join(out) + "\n"


def main(argv):
    fns = {"trace": trace, "traffic": traffic, "stats": stats, "pmc": pmc}
    if len(argv) != 5 or argv[1] not in fns:
        raise SystemExit(__doc__)
    sys.stdout.write(fns[argv[1]](argv[2], argv[3], argv[4]))


if __name__ == "__main__":
    main(sys.argv)
