"""HBM traffic of the library's kernels from rocprofv3 counter runs.

Two counter passes of the same bench command (one with FETCH_SIZE, one with WRITE_SIZE, both in
KiB per dispatch) are turned into bytes per launch.  Each counter is scaled by what it reads for
a plain device copy of a known size that bench.py runs in the same process (--copy-mib), so the
result is in the copy's units: bytes that a plain copy would move.  The summary goes to
profiles/traffic_<workload>.json (read by bench.py, valid only for the kernel sources it was
taken from)
and a short markdown table.

Usage:
  python -m jagged_attention_amd.traffic FETCH_CSV WRITE_CSV --copy-mib N --workload NAME \
      --command "the bench command the counters were taken on"
"""
from __future__ import annotations

import argparse
import collections
import csv
import hashlib
import json
import os
import re

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


# timing name -> the source file that defines the kernel
KERNEL_SOURCE = {"jfa_bwd_kvq": "bwd_inst.hip", "jfa_bwd_dkdv": "bwd_inst.hip",
                 "jfa_bwd_dq": "bwd_inst.hip", "jfa_dbias_dq": "bwd_inst.hip",
                 "jfa_bwd_kvq_mxfp8": "bwd_inst.hip", "jfa_bwd_dkdv_mxfp8": "bwd_inst.hip",
                 "jfa_bwd_dq_mxfp8": "bwd_inst.hip",
                 "jfa_fwd_bf16": "fwd.hip",
                 "jfa_fwd_mxfp8": "fwd.hip", "jfa_fwd_combine": "fwd.hip",
                 "jfa_schedule": "sched.hip", "jfa_offsets": "sched.hip",
                 "jfa_quant_mxfp8": "quant.hip", "jfa_fwd_f32": "f32.hip",
                 "jfa_bwd_dq_f32": "f32.hip", "jfa_bwd_dkdv_f32": "f32.hip"}
# what every kernel's code and launch configuration also depend on
SHARED_SOURCES = ("jfa_device.h", "jfa_internal.h", "api.cpp")


def source_hash(kernel: str | None = None) -> str:
    """Hash of the sources a kernel is built and launched from (its own file plus the shared
    headers and the launcher), or of every source when `kernel` is None: counters describe one
    version of that code."""
    h = hashlib.sha256()
    csrc = os.path.join(HERE, "csrc")
    if kernel is None:
        files = sorted(os.listdir(csrc))
    else:
        files = sorted({KERNEL_SOURCE.get(kernel, "")} - {""} | set(SHARED_SOURCES))
        if kernel not in KERNEL_SOURCE:
            files = sorted(os.listdir(csrc))
    for f in files:
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode())
            h.update(fh.read())
    return h.hexdigest()[:16]


# device kernel name -> the timing name bench.py reports
def _targs(kernel: str, name: str) -> list:
    m = re.search(name + r"<([^>]*)>", kernel)
    return [x.strip() for x in m.group(1).split(",")] if m else []


def timing_name(kernel: str) -> str | None:
    k = kernel
    for base, tname in (("bwd_kvq_kernel", "jfa_bwd_kvq"), ("bwd_kv_kernel", "jfa_bwd_dkdv"),
                        ("bwd_q_db_kernel", "jfa_dbias_dq"), ("bwd_q_kernel", "jfa_bwd_dq"),
                        ("bwd_q1_kernel", "jfa_bwd_dq")):
        if base in k:
            a = _targs(k, base)          # <D, NW, MODE, BIAS, WIN, FP8>
            return tname + ("_mxfp8" if len(a) >= 6 and a[5] == "true" else "")
    if "combine_kernel" in k:
        return "jfa_fwd_combine"
    if "fwd_kernel" in k:
        a = _targs(k, "fwd_kernel")      # <D, NW, MODE, BIAS, FP8, WIN>
        return "jfa_fwd_mxfp8" if len(a) >= 5 and a[4] == "true" else "jfa_fwd_bf16"
    if "schedule_kernel" in k:
        return "jfa_schedule"
    if "lengths_to_offsets" in k:
        return "jfa_offsets"
    if "rmsnorm_quant" in k:
        return "jfa_norm_quant_mxfp8"
    if "quantize" in k or "quant" in k:
        return "jfa_quant_mxfp8"
    if "dbias_rows" in k or "dbias_chunks" in k:
        return "jfa_dbias_reduce"
    if "zero_u16" in k:
        return "jfa_dbias_zero"
    if "copyBuffer" in k:
        return "copy"
    return None


def read_counter(path: str, counter: str):
    """{kernel name: [value per dispatch]} for one counter from a rocprofv3 counter CSV."""
    out = collections.defaultdict(list)
    with open(path) as fh:
        for r in csv.DictReader(fh):
            if r["Counter_Name"] != counter:
                continue
            out[r["Kernel_Name"]].append(float(r["Counter_Value"]))
    return out


def summarize(fetch_csv: str, write_csv: str, copy_bytes: int):
    fetch = read_counter(fetch_csv, "FETCH_SIZE")
    write = read_counter(write_csv, "WRITE_SIZE")

    def by_name(d):
        agg = collections.defaultdict(list)
        for k, v in d.items():
            n = timing_name(k)
            if n:
                agg[n].extend(v)
        return agg

    f, w = by_name(fetch), by_name(write)
    # the calibration copy: the largest copy dispatch (reads and writes copy_bytes each)
    cf = max(f.get("copy", [0.0]))
    cw = max(w.get("copy", [0.0]))
    if cf <= 0 or cw <= 0:
        raise SystemExit("no calibration copy found in the counter files")
    kf = copy_bytes / (cf * 1024.0)
    kw = copy_bytes / (cw * 1024.0)
    kernels = {}
    for name in sorted(set(f) | set(w)):
        if name == "copy":
            continue
        fv, wv = f.get(name, []), w.get(name, [])
        fb = (sum(fv) / len(fv)) * 1024.0 * kf if fv else 0.0
        wb = (sum(wv) / len(wv)) * 1024.0 * kw if wv else 0.0
        kernels[name] = dict(fetch_bytes=round(fb), write_bytes=round(wb),
                             bytes_per_launch=round(fb + wb), dispatches=len(fv),
                             source_hash=source_hash(name))
    calib = dict(copy_bytes=copy_bytes, fetch_kib=cf, write_kib=cw, fetch_factor=round(kf, 4),
                 write_factor=round(kw, 4))
    return kernels, calib


def file_tag(workload: str) -> str:
    """The workload name as used in profile file names."""
    return re.sub(r"[^a-z0-9]+", "_", workload.lower()).strip("_")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("fetch_csv")
    ap.add_argument("write_csv")
    ap.add_argument("--copy-mib", type=int, required=True)
    ap.add_argument("--workload", required=True)
    ap.add_argument("--command", required=True)
    ap.add_argument("--out", default=os.path.join(ROOT, "profiles"))
    a = ap.parse_args()
    kernels, calib = summarize(a.fetch_csv, a.write_csv, a.copy_mib << 20)
    rec = dict(source_hash=source_hash(), workload=a.workload, command=a.command,
               calibration=calib, kernels=kernels)
    with open(os.path.join(a.out, f"traffic_{file_tag(a.workload)}.json"), "w") as fh:
        json.dump(rec, fh, indent=1)
    lines = [f"# HBM traffic per launch: {a.workload}", "",
             f"Counters: rocprofv3 --pmc FETCH_SIZE, then --pmc WRITE_SIZE, each on `{a.command}`.",
             f"Calibration: a {a.copy_mib} MiB device copy in the same run read FETCH_SIZE "
             f"{calib['fetch_kib']:.0f} KiB and WRITE_SIZE {calib['write_kib']:.0f} KiB; factors "
             f"{calib['fetch_factor']} and {calib['write_factor']} convert the counters to bytes.",
             f"Kernel sources (all files): {rec['source_hash']}; per kernel in the .json beside "
             f"this file.", "",
             "| kernel | fetch MB | write MB | total MB / launch | dispatches |",
             "|---|---|---|---|---|"]
    for n, e in kernels.items():
        lines.append(f"| {n} | {e['fetch_bytes'] / 1e6:.1f} | {e['write_bytes'] / 1e6:.1f} | "
                     f"{e['bytes_per_launch'] / 1e6:.1f} | {e['dispatches']} |")
    with open(os.path.join(a.out, f"traffic_{file_tag(a.workload)}.md"), "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print(json.dumps(rec, indent=1))


if __name__ == "__main__":
    main()
