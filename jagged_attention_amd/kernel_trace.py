"""Per-kernel durations of the library's kernels from a rocprofv3 --kernel-trace run.

Reads the run's kernel_trace.csv, groups the dispatches by the timing name bench.py reports
(jagged_attention_amd.traffic.timing_name), and writes profiles/<workload>_kernel_trace.md: calls,
average and median duration, and each kernel's share of the library's time.

Usage:
  python -m jagged_attention_amd.kernel_trace TRACE_CSV --workload NAME --command CMD \
      [--bench-json BENCH_JSON]
With --bench-json (the bench line the traced command printed), the in-bench HIP-event averages
of the same run are listed beside the trace's.
"""
from __future__ import annotations

import argparse
import collections
import csv
import json
import os

import numpy as np

from jagged_attention_amd.traffic import ROOT, file_tag, timing_name


def read(path):
    """{timing name: [duration in us per dispatch]} plus one full kernel name per timing name."""
    out = collections.defaultdict(list)
    full = {}
    with open(path) as fh:
        for r in csv.DictReader(fh):
            n = timing_name(r["Kernel_Name"])
            if not n or n == "copy":
                continue
            out[n].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1000.0)
            k = r["Kernel_Name"].replace("jfa::(anonymous namespace)::", "").replace("void ", "")
            full.setdefault(n, k.split("(")[0])
    return out, full


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("trace_csv")
    ap.add_argument("--workload", required=True)
    ap.add_argument("--command", required=True)
    ap.add_argument("--bench-json")
    ap.add_argument("--out", default=os.path.join(ROOT, "profiles"))
    a = ap.parse_args()
    durs, full = read(a.trace_csv)
    total = sum(sum(v) for v in durs.values())
    bench = None
    if a.bench_json:
        with open(a.bench_json) as fh:
            bench = json.loads(fh.read().strip().splitlines()[-1])
    lines = [f"# Kernel trace: {a.workload}", "",
             "Command (from the repository root, on one MI355X):", "",
             f"    {a.command}", "",
             "Every dispatch of the run is listed: warm-up, the timed steps, the graph capture "
             "check and replays, and the per-kernel event timing (the profiler serialises the "
             "launches).", "",
             "| Kernel | Instance | Calls | Avg (us) | Median (us) | Share of library time |",
             "|---|---|---|---|---|---|"]
    for n in sorted(durs, key=lambda k: -sum(durs[k])):
        v = np.array(durs[n])
        lines.append(f"| {n} | `{full[n][:60]}` | {len(v)} | {v.mean():.1f} | "
                     f"{np.median(v):.1f} | {100 * v.sum() / total:.1f}% |")
    if bench:
        kt = bench.get("kernels", {})
        lines += ["", "In-bench HIP-event averages of the same run (us): " +
                  ", ".join(f"{k} {1000 * e['avg_ms']:.1f}" for k, e in kt.items()) + "."]
    path = os.path.join(a.out, f"{file_tag(a.workload)}_kernel_trace.md")
    with open(path, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


if __name__ == "__main__":
    main()
