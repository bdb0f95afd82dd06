"""Builds libjfa.so (HIP kernels for gfx950 + the C ABI) in-tree with hipcc.

Usage: python -m jagged_attention_amd.build [--incremental]   (or build() from Python).
Every HIP source is compiled separately (in parallel) under _build/, then linked.  The MFMA
backward (bwd_inst.hip) is compiled once per (head dim, mode, input format), so its instances
build in parallel.  --incremental reuses objects newer than every source and header they depend on.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libjfa.so")
BUILD_DIR = os.path.join(ROOT, "_build")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-I", os.path.join(ROOT, "include"),
          # packed fp32 VALU forms are kept out of every device build
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-Wno-unused-command-line-argument"]


# translation units compiled once per variant: source -> [(object suffix, extra flags)]
VARIANTS = {
    "bwd_inst.hip": [(f"d{d}_m{m}_f{f}", [f"-DJFA_BWD_D={d}", f"-DJFA_BWD_MODE={m}",
                                          f"-DJFA_BWD_FP8={f}"])
                     for d in (128, 64) for m in (0, 1, 2) for f in (0, 1)],
}


def sources():
    """(source, object name, extra flags) of every translation unit."""
    names = sorted(f for f in os.listdir(CSRC) if f.endswith((".hip", ".cpp")))
    out = []
    for f in names:
        src = os.path.join(CSRC, f)
        for suffix, flags in VARIANTS.get(f, [("", [])]):
            out.append((src, f + (f".{suffix}" if suffix else "") + ".o", flags))
    return out


def _deps_mtime(src: str) -> float:
    deps = [src, os.path.join(ROOT, "include", "jfa.h")]
    deps += [os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".h")]
    return max(os.path.getmtime(p) for p in deps)


def _compile(unit, incremental: bool = False) -> str:
    src, oname, flags = unit
    obj = os.path.join(BUILD_DIR, oname)
    if incremental and os.path.exists(obj) and os.path.getmtime(obj) > _deps_mtime(src):
        return obj
    cmd = [HIPCC, *COMMON, *flags, "-c", src, "-o", obj]
    if src.endswith(".cpp"):
        cmd = [HIPCC, "-O2", "-std=c++17", "-fPIC", "-I", os.path.join(ROOT, "include"), "-c", src,
               "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    msg = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{msg}")
    if msg.strip():
        sys.stderr.write(msg + "\n")
    return obj


def build(jobs: int | None = None, incremental: bool = False) -> str:
    """Compiles every source and links jagged_attention_amd/libjfa.so; returns its path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    units = sources()
    jobs = jobs or min(len(units), max(1, (os.cpu_count() or 4)))
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda u: _compile(u, incremental), units))
    tmp = OUT + f".tmp{os.getpid()}"
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}{r.stderr}")
    os.replace(tmp, OUT)
    return OUT


if __name__ == "__main__":
    print(build(incremental="--incremental" in sys.argv[1:]))
