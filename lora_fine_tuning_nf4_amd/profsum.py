"""Text summaries of rocprofv3 CSV output for the forward GEMM the benchmark reports.

    python -m lora_fine_tuning_nf4_amd.profsum trace   TRACE_DIR BENCH_JSON  "<command>"
    python -m lora_fine_tuning_nf4_amd.profsum traffic FETCH_DIR WRITE_DIR   "<command>"
    python -m lora_fine_tuning_nf4_amd.profsum stats   TRACE_DIR -           "<command>"

``trace`` reads ``*_kernel_stats.csv`` and ``*_kernel_trace.csv`` of a ``--kernel-trace
--stats -f csv`` run of bench.py and prints the per-kernel table plus the average
duration of the dominant launch (the gate|up forward: grid = 896 workgroups x 256
threads at the 8B shape) over the benchmark's timed launches, beside the benchmark's own
HIP-event average from the same run.

``stats`` prints the per-kernel table of a kernel-trace run (every kernel, by total time).

``traffic`` reads the ``*_counter_collection.csv`` of two ``--pmc FETCH_SIZE`` and
``--pmc WRITE_SIZE`` runs and scales each counter by what it reads for the benchmark's
calibration kernel (a float32 elementwise copy of 256 MiB in, 256 MiB out), giving HBM
bytes per launch of the dominant kernel.  The printed ``kernel_source_sha256`` ties the
figures to the kernel sources they were taken on.
"""
from __future__ import annotations

import csv
import glob
import json
import os
import sys

DOM_NAME = "k_fwd_nf4<256, 4>"
DOM_GRID = (768 + 256) * 256  # threads: 768 tiles of 256 x 256 and 256 tiles of 128 x 256
CAL_NAME = "neg_kernel"
CAL_BYTES = 256 << 20


def _one(pattern: str) -> str:
    hits = sorted(glob.glob(pattern, recursive=True))
    if not hits:
        raise SystemExit(f"no file matches {pattern}")
    return hits[0]


def _short(name: str, n: int = 70) -> str:
    return name if len(name) <= n else name[: n - 3] + "..."


def trace(trace_dir: str, bench_json: str, command: str) -> str:
    stats = list(csv.DictReader(open(_one(os.path.join(trace_dir, "**", "*kernel_stats.csv")))))
    rows = list(csv.DictReader(open(_one(os.path.join(trace_dir, "**", "*kernel_trace.csv")))))
    bench = None
    with open(bench_json) as fh:
        for line in fh:
            line = line.strip()
            if line.startswith("{") and '"roofline"' in line:
                bench = json.loads(line)
    out = [f"# rocprofv3 kernel trace: {command}", ""]
    out.append(f"{'kernel':72s} {'calls':>6s} {'avg_us':>10s} {'min_us':>9s} {'max_us':>9s} {'share%':>7s}")
    for r in stats[:16]:
        out.append(f"{_short(r['Name'], 72):72s} {int(r['Calls']):6d} {float(r['AverageNs']) / 1e3:10.2f} "
                   f"{float(r['MinNs']) / 1e3:9.2f} {float(r['MaxNs']) / 1e3:9.2f} {float(r['Percentage']):7.2f}")
    dom = sorted((int(r["Start_Timestamp"]), int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
                 for r in rows if DOM_NAME in r["Kernel_Name"] and int(r["Grid_Size_X"]) == DOM_GRID)
    out.append("")
    out.append(f"dominant launch: {DOM_NAME} with grid {DOM_GRID} (gate|up forward, M=2048 N=28672 K=4096)")
    out.append(f"  dispatches in the trace: {len(dom)}")
    if bench is not None and dom:
        # the bench's warm-up steps come first, then its timed steps
        n = int(bench["roofline"]["launches_timed"])
        skip = int(bench["warmup"]) * (n // int(bench["steps"]))
        timed = [d for _, d in dom[skip:skip + n]]
        avg = sum(timed) / len(timed) / 1e6
        out.append(f"  timed-region dispatches (#{skip}..#{skip + n - 1}): avg {avg:.4f} ms, "
                   f"min {min(timed) / 1e6:.4f} ms, max {max(timed) / 1e6:.4f} ms")
        out.append(f"  bench.py HIP-event average in the same run: {bench['roofline']['avg_launch_ms']:.4f} ms "
                   f"(ratio {bench['roofline']['avg_launch_ms'] / avg:.3f})")
        out.append(f"  bench.py ms_per_step {bench['ms_per_step']}, value {bench['value']} {bench['unit']}")
    return "\n".join(out) + "\n"


def _counter(dir_: str, counter: str):
    rows = list(csv.DictReader(open(_one(os.path.join(dir_, "**", "*counter_collection.csv")))))
    dom = [float(r["Counter_Value"]) for r in rows
           if r["Counter_Name"] == counter and DOM_NAME in r["Kernel_Name"] and int(r["Grid_Size"]) == DOM_GRID]
    cal = [float(r["Counter_Value"]) for r in rows if r["Counter_Name"] == counter and CAL_NAME in r["Kernel_Name"]]
    if not dom or not cal:
        raise SystemExit(f"{counter}: dominant or calibration kernel missing in {dir_}")
    return sum(dom) / len(dom), len(dom), cal[-1]


def traffic(fetch_dir: str, write_dir: str, command: str) -> str:
    sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
    import bench  # the hash of the kernel sources, defined once

    f_dom, f_n, f_cal = _counter(fetch_dir, "FETCH_SIZE")
    w_dom, w_n, w_cal = _counter(write_dir, "WRITE_SIZE")
    f_fac = f_cal * 1024.0 / CAL_BYTES
    w_fac = w_cal * 1024.0 / CAL_BYTES
    fetch_b = f_dom * 1024.0 / f_fac
    write_b = w_dom * 1024.0 / w_fac
    lines = [
        f"# HBM traffic per launch of {DOM_NAME} grid {DOM_GRID} (gate|up forward, M=2048 N=28672 K=4096)",
        f"# command: {command}",
        "# each counter is scaled by its reading for the calibration copy (256 MiB read, 256 MiB written)",
        f"kernel_source_sha256: {bench.kernel_source_hash()}",
        f"fetch_kib_per_launch: {f_dom:.1f}",
        f"fetch_launches: {f_n}",
        f"write_kib_per_launch: {w_dom:.1f}",
        f"write_launches: {w_n}",
        f"calibration_fetch_kib: {f_cal:.1f}",
        f"calibration_write_kib: {w_cal:.1f}",
        f"fetch_scale: {f_fac:.5f}",
        f"write_scale: {w_fac:.5f}",
        f"fetch_bytes_per_launch: {fetch_b:.0f}",
        f"write_bytes_per_launch: {write_b:.0f}",
        f"traffic_bytes_per_launch: {fetch_b + write_b:.0f}",
        f"algorithmic_bytes_per_launch: {bench.fwd_bytes(__import__('synthgen').WORKLOADS['llama8b'], ('gate', 'up'))}",
    ]
    return "\n".join(lines) + "\n"


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
    fns = {"trace": trace, "traffic": traffic, "stats": stats}
    if len(argv) != 5 or argv[1] not in fns:
        raise SystemExit(__doc__)
    sys.stdout.write(fns[argv[1]](argv[2], argv[3], argv[4]))


if __name__ == "__main__":
    main(sys.argv)
