"""Summaries of rocprofv3 runs of bench.py, as short text for ``profiles/``.

rocprofv3 writes, per run directory, ``*_kernel_stats.csv`` (``--kernel-trace
--stats``) and ``*_counter_collection.csv`` (``--pmc``). This module reduces
them to the figures the benchmark and the design notes use:

* the kernel-trace table (calls, average / min / max duration per kernel);
* the durations of the named kernel over exactly the bench run's timed
  steps (its dispatches after the warmup ones, from the per-dispatch
  trace), as median / min / p90 / average, and the rate at the median from
  the algorithmic work of one launch, beside the bench line's own figures
  (``--bench-log``: the file holding the JSON line that run printed);
* HBM traffic per attention launch: FETCH_SIZE and WRITE_SIZE (KiB per
  dispatch) averaged over the attention dispatches, each scaled by the
  factor that makes the same counter read exactly the known byte count of a
  plain copy kernel (``bench.py --copy-calibration MIB``: the last three
  dispatches of that run each read and write MIB MiB).

Usage (from the repository root, after the rocprofv3 runs)::

    python -m accelerator_programming_amd.profsummary --workload C4 \\
        --kernel attn_fwd_kernel --trace DIR --fetch DIR --write DIR \\
        --copy-fetch DIR --copy-write DIR --copy-mib 1024 \\
        --commands FILE --out profiles/attn_fwd_C4

writes ``<out>_kernel_trace.txt`` and ``<out>_traffic.json`` (and, with
``--counters DIR ...``, ``<out>_counters.txt``).
"""
from __future__ import annotations

import argparse
import csv
import glob
import json
import os
import sys


def _one(pattern: str) -> str:
    hits = sorted(glob.glob(pattern, recursive=True))
    if not hits:
        raise FileNotFoundError(pattern)
    return hits[0]


def kernel_stats(run_dir: str):
    """Rows of the kernel-trace statistics, longest total time first."""
    path = _one(os.path.join(run_dir, "**", "*kernel_stats.csv"))
    rows = list(csv.DictReader(open(path)))
    rows.sort(key=lambda r: -float(r["TotalDurationNs"]))
    return rows


def counter_per_dispatch(run_dir: str, counter: str, kernel_substr: str | None):
    """[(dispatch id, value)] of one counter, for dispatches whose kernel name
    contains kernel_substr (all dispatches when None), in dispatch order."""
    path = _one(os.path.join(run_dir, "**", "*counter_collection.csv"))
    out = {}
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] != counter:
            continue
        if kernel_substr and kernel_substr not in r["Kernel_Name"]:
            continue
        d = int(r["Dispatch_Id"])
        out[d] = out.get(d, 0.0) + float(r["Counter_Value"])
    return sorted(out.items())


def traffic(fetch_dir, write_dir, copy_fetch_dir, copy_write_dir, copy_mib, kernel_substr):
    """HBM bytes per attention launch from FETCH_SIZE / WRITE_SIZE (KiB per
    dispatch), each scaled by the copy-kernel calibration."""
    copy_bytes = copy_mib * (1 << 20)
    cf = [v for _, v in counter_per_dispatch(copy_fetch_dir, "FETCH_SIZE", None)[-3:]]
    cw = [v for _, v in counter_per_dispatch(copy_write_dir, "WRITE_SIZE", None)[-3:]]
    f_scale = copy_bytes / (sum(cf) / len(cf) * 1024.0)
    w_scale = copy_bytes / (sum(cw) / len(cw) * 1024.0)
    af = [v for _, v in counter_per_dispatch(fetch_dir, "FETCH_SIZE", kernel_substr)]
    aw = [v for _, v in counter_per_dispatch(write_dir, "WRITE_SIZE", kernel_substr)]
    fetch_kib = sum(af) / len(af)
    write_kib = sum(aw) / len(aw)
    return {
        "fetch_kib_per_dispatch": fetch_kib,
        "write_kib_per_dispatch": write_kib,
        "copy_fetch_kib_per_dispatch": sum(cf) / len(cf),
        "copy_write_kib_per_dispatch": sum(cw) / len(cw),
        "copy_bytes": copy_bytes,
        "fetch_scale": f_scale,
        "write_scale": w_scale,
        "fetch_bytes_per_launch": fetch_kib * 1024.0 * f_scale,
        "write_bytes_per_launch": write_kib * 1024.0 * w_scale,
        "bytes_per_launch": fetch_kib * 1024.0 * f_scale + write_kib * 1024.0 * w_scale,
        "dispatches": [len(af), len(aw)],
    }


def dispatch_ns(run_dir: str, kernel_substr: str):
    """Durations (ns) of the dispatches whose kernel name contains
    kernel_substr, in dispatch order, from ``*_kernel_trace.csv``."""
    path = _one(os.path.join(run_dir, "**", "*kernel_trace.csv"))
    rows = [r for r in csv.DictReader(open(path)) if kernel_substr in r["Kernel_Name"]]
    rows.sort(key=lambda r: int(r["Dispatch_Id"]))
    return [int(r["End_Timestamp"]) - int(r["Start_Timestamp"]) for r in rows]


def bench_line(path: str) -> dict:
    """The last JSON line a bench.py run printed."""
    line = None
    for x in open(path):
        if x.startswith("{"):
            line = x
    if line is None:
        raise ValueError("no bench line in %s" % path)
    return json.loads(line)


def timed_window(ns, line: dict) -> list[str]:
    """Statistics of the bench run's timed launches (the dispatches after
    its warmup ones) and the rate at their median, from the work of one
    launch that the bench line implies (achieved x its average time)."""
    w, k = int(line["warmup"]), int(line["steps"])
    xs = sorted(ns[w:w + k])
    if len(xs) < k:
        return ["(the trace holds %d dispatches of the kernel, fewer than warmup %d + steps %d)"
                % (len(ns), w, k)]
    r = line["roofline"]
    unit = r["unit"]
    work = r["achieved"] * r["kernel_ms_avg"]  # unit x ms per launch
    med, avg = xs[len(xs) // 2], sum(xs) / len(xs)
    p90 = xs[min(len(xs) - 1, -(-9 * len(xs) // 10) - 1)]
    return [
        "Timed launches: dispatches %d .. %d of the kernel (after %d warmup ones)" % (w + 1, w + k, w),
        "  median %.0f ns, min %d ns, p90 %d ns, average %.0f ns" % (med, xs[0], p90, avg),
        "  at the median: %.2f %s; at the average: %.2f %s (algorithmic work per launch)"
        % (work / (med * 1e-6), unit, work / (avg * 1e-6), unit),
        "Bench line of this run (HIP events, profiler attached): value %s %s, ms_per_step %s,"
        % (line["value"], line["unit"], line["ms_per_step"]),
        "  achieved %s %s (frac %s), kernel_ms median %s min %s p90 %s"
        % (r["achieved"], unit, r["frac"], r.get("kernel_ms_median"), r.get("kernel_ms_min"),
           r.get("kernel_ms_p90")),
    ]


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--workload", required=True)
    ap.add_argument("--kernel", required=True, help="substring of the attention kernel's name")
    ap.add_argument("--trace", required=True)
    ap.add_argument("--fetch")
    ap.add_argument("--write")
    ap.add_argument("--copy-fetch")
    ap.add_argument("--copy-write")
    ap.add_argument("--copy-mib", type=int, default=1024)
    ap.add_argument("--counters", nargs="*", default=[],
                    help="further --pmc run directories: every counter averaged per dispatch")
    ap.add_argument("--commands", help="text file with the rocprofv3 command lines used")
    ap.add_argument("--kernel-sha", help="source hash the counters were taken on")
    ap.add_argument("--bench-log", help="output of the traced bench.py run (its JSON line)")
    ap.add_argument("--out", required=True, help="output prefix, e.g. profiles/attn_fwd_C4")
    a = ap.parse_args(argv)

    cmds = open(a.commands).read().strip() if a.commands else "(not recorded)"
    rows = kernel_stats(a.trace)
    lines = ["rocprofv3 kernel trace, workload %s" % a.workload, "", "Commands:", cmds, "",
             "%-60s %6s %14s %14s %14s %8s" % ("kernel", "calls", "avg ns", "min ns", "max ns", "% time")]
    for r in rows[:8]:
        name = r["Name"]
        lines.append("%-60s %6s %14.0f %14s %14s %8s" % (
            (name[:57] + "...") if len(name) > 60 else name, r["Calls"], float(r["AverageNs"]),
            r["MinNs"], r["MaxNs"], r["Percentage"]))
    if a.bench_log:
        lines += [""] + timed_window(dispatch_ns(a.trace, a.kernel), bench_line(a.bench_log))
    with open(a.out + "_kernel_trace.txt", "w") as f:
        f.write("\n".join(lines) + "\n")

    if a.counters:
        out = ["rocprofv3 counters per %s dispatch (mean over dispatches), workload %s" % (
            a.kernel, a.workload), "", "Commands:", cmds, ""]
        for d in a.counters:
            path = _one(os.path.join(d, "**", "*counter_collection.csv"))
            names = sorted({r["Counter_Name"] for r in csv.DictReader(open(path))})
            for n in names:
                v = [x for _, x in counter_per_dispatch(d, n, a.kernel)]
                if v:
                    out.append("%-28s %.6g" % (n, sum(v) / len(v)))
        with open(a.out + "_counters.txt", "w") as f:
            f.write("\n".join(out) + "\n")

    if a.fetch and a.write and a.copy_fetch and a.copy_write:
        t = traffic(a.fetch, a.write, a.copy_fetch, a.copy_write, a.copy_mib, a.kernel)
        t.update({"workload": a.workload, "kernel": a.kernel, "kernel_sha": a.kernel_sha,
                  "commands": cmds.splitlines()})
        with open(a.out + "_traffic.json", "w") as f:
            json.dump(t, f, indent=1)
            f.write("\n")
    return 0


if __name__ == "__main__":
    sys.exit(main())
