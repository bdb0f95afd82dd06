"""Issue-level counters of the library's kernels from two rocprofv3 --pmc passes.

Pass A: SQ_VALU_MFMA_BUSY_CYCLES SQ_BUSY_CU_CYCLES SQ_ACTIVE_INST_VALU SQ_INSTS_MFMA SQ_INSTS_VALU
        SQ_LDS_IDX_ACTIVE SQ_LDS_BANK_CONFLICT GRBM_GUI_ACTIVE
Pass B: SQ_WAVES SQ_WAVE_CYCLES SQ_WAIT_ANY SQ_WAIT_INST_ANY SQ_ACTIVE_INST_ANY SQ_INSTS_SALU
        SQ_ACTIVE_INST_LDS GRBM_GUI_ACTIVE

Per kernel (averaged over its dispatches): GRBM_GUI_ACTIVE is summed over the 8 XCDs, so one XCD's
busy cycles are an eighth of it; MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (cycles x 1024 SIMDs);
LDS active and bank-conflict stalls = SQ_LDS_IDX_ACTIVE, SQ_LDS_BANK_CONFLICT / (cycles x 256
CUs); VALU instructions per MFMA = SQ_INSTS_VALU / SQ_INSTS_MFMA; waiting = SQ_WAIT_ANY /
SQ_WAVE_CYCLES.

Optional stall passes (--stalls PASS_C_CSV PASS_D_CSV):
Pass C: SQ_WAVE_CYCLES SQ_WAIT_INST_ANY SQ_WAIT_ANY SQ_ACTIVE_INST_ANY SQ_ACTIVE_INST_VALU
        SQ_ACTIVE_INST_LDS SQ_VMEM_TA_ADDR_FIFO_FULL SQ_LDS_CMD_FIFO_FULL GRBM_GUI_ACTIVE
Pass D: SQ_ACTIVE_INST_VMEM SQ_ACTIVE_INST_MISC SQ_ACTIVE_INST_SCA SQ_VMEM_TA_CMD_FIFO_FULL
        SQ_LDS_DATA_FIFO_FULL SQ_WAIT_INST_LDS SQ_VALU_MFMA_COEXEC_CYCLES SQ_INST_LEVEL_LDS
        GRBM_GUI_ACTIVE
A wave's time splits into issuing (SQ_ACTIVE_INST_ANY), waiting on a memory counter
(SQ_WAIT_ANY) and waiting for an issue slot or a dependency (SQ_WAIT_INST_ANY), each over
SQ_WAVE_CYCLES (the same units); the per-type issue shares are over SQ_WAVE_CYCLES too.  The
FIFO-full counters are reported per CU as a share of the kernel's cycles, taking them in the
same 4-cycle units as SQ_WAVE_CYCLES.

Usage:
  python -m jagged_attention_amd.counters PASS_A_CSV PASS_B_CSV --workload NAME --command CMD \
      [--stalls PASS_C_CSV PASS_D_CSV --stall-command CMD]
writes profiles/<workload>_utilisation.md (and profiles/<workload>_stalls.md).
"""
from __future__ import annotations

import argparse
import collections
import csv
import os

from jagged_attention_amd.traffic import ROOT, file_tag, timing_name

XCDS, SIMDS, CUS = 8, 1024, 256


def read(path):
    """{timing name: {counter: [value per dispatch]}}."""
    out = collections.defaultdict(lambda: collections.defaultdict(list))
    with open(path) as fh:
        for r in csv.DictReader(fh):
            n = timing_name(r["Kernel_Name"])
            if not n or n == "copy":
                continue
            out[n][r["Counter_Name"]].append(float(r["Counter_Value"]))
    return out


def mean(v):
    return sum(v) / len(v) if v else 0.0


def summarize(path_a, path_b):
    a = read(path_a)
    b = read(path_b)
    rows = {}
    for n in sorted(set(a) | set(b)):
        ca, cb = a.get(n, {}), b.get(n, {})
        cyc = mean(ca.get("GRBM_GUI_ACTIVE", [])) / XCDS
        mfma = mean(ca.get("SQ_INSTS_MFMA", []))
        rows[n] = dict(
            cycles=cyc,
            mfma_busy=mean(ca.get("SQ_VALU_MFMA_BUSY_CYCLES", [])) / (cyc * SIMDS) if cyc else 0,
            lds_active=mean(ca.get("SQ_LDS_IDX_ACTIVE", [])) / (cyc * CUS) if cyc else 0,
            lds_conflict=mean(ca.get("SQ_LDS_BANK_CONFLICT", [])) / (cyc * CUS) if cyc else 0,
            valu_per_mfma=mean(ca.get("SQ_INSTS_VALU", [])) / mfma if mfma else 0,
            waves=mean(cb.get("SQ_WAVES", [])),
            waiting=(mean(cb.get("SQ_WAIT_ANY", [])) / mean(cb.get("SQ_WAVE_CYCLES", []))
                     if mean(cb.get("SQ_WAVE_CYCLES", [])) else 0),
            dispatches=len(ca.get("GRBM_GUI_ACTIVE", [])))
    return rows


def summarize_stalls(path_c, path_d):
    c = read(path_c)
    d = read(path_d)
    rows = {}
    for n in sorted(set(c) | set(d)):
        cc, cd = c.get(n, {}), d.get(n, {})
        wc = mean(cc.get("SQ_WAVE_CYCLES", []))
        cyc = mean(cc.get("GRBM_GUI_ACTIVE", [])) / XCDS
        if not wc or not cyc:
            continue
        share = lambda src, k: mean(src.get(k, [])) / wc
        per_cu = lambda src, k: mean(src.get(k, [])) * 4 / (cyc * CUS)
        rows[n] = dict(
            issuing=share(cc, "SQ_ACTIVE_INST_ANY"), waitcnt=share(cc, "SQ_WAIT_ANY"),
            wait_issue=share(cc, "SQ_WAIT_INST_ANY"), valu=share(cc, "SQ_ACTIVE_INST_VALU"),
            lds=share(cc, "SQ_ACTIVE_INST_LDS"), sca=share(cd, "SQ_ACTIVE_INST_SCA"),
            vmem=share(cd, "SQ_ACTIVE_INST_VMEM"), wait_lds=share(cd, "SQ_WAIT_INST_LDS"),
            ta_addr_full=per_cu(cc, "SQ_VMEM_TA_ADDR_FIFO_FULL"),
            ta_cmd_full=per_cu(cd, "SQ_VMEM_TA_CMD_FIFO_FULL"),
            lds_data_full=per_cu(cd, "SQ_LDS_DATA_FIFO_FULL"),
            dispatches=len(cc.get("GRBM_GUI_ACTIVE", [])))
    return rows


def write_stalls(rows, workload, command, out):
    lines = [f"# Where the waves' time goes: {workload}", "",
             "Two more counter passes of the same command (see jagged_attention_amd/counters.py "
             "for the counter sets and the formulas):", "", f"    {command}", "",
             "Shares of wave time: issuing an instruction, waiting on a memory counter "
             "(s_waitcnt), waiting for an issue slot or a dependency; then the issue shares by "
             "instruction type and the share of each CU's cycles with a texture-address (TA) or "
             "LDS FIFO full.", "",
             "| Kernel | Issuing | Waiting on memory | Waiting to issue | VALU+MFMA issue | "
             "LDS issue | VMEM issue | Scalar issue | Waiting to issue LDS | TA addr FIFO full | "
             "TA cmd FIFO full | LDS data FIFO full |",
             "|---|---|---|---|---|---|---|---|---|---|---|---|"]
    pct = lambda x: f"{100 * x:.1f}%"
    for n, r in rows.items():
        lines.append(f"| {n} | {pct(r['issuing'])} | {pct(r['waitcnt'])} | "
                     f"{pct(r['wait_issue'])} | {pct(r['valu'])} | {pct(r['lds'])} | "
                     f"{pct(r['vmem'])} | {pct(r['sca'])} | {pct(r['wait_lds'])} | "
                     f"{pct(r['ta_addr_full'])} | {pct(r['ta_cmd_full'])} | "
                     f"{pct(r['lds_data_full'])} |")
    path = os.path.join(out, f"{file_tag(workload)}_stalls.md")
    with open(path, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("pass_a")
    ap.add_argument("pass_b")
    ap.add_argument("--workload", required=True)
    ap.add_argument("--command", required=True)
    ap.add_argument("--stalls", nargs=2, metavar=("PASS_C", "PASS_D"))
    ap.add_argument("--stall-command")
    ap.add_argument("--out", default=os.path.join(ROOT, "profiles"))
    a = ap.parse_args()
    if a.stalls:
        write_stalls(summarize_stalls(*a.stalls), a.workload, a.stall_command or a.command,
                     a.out)
    rows = summarize(a.pass_a, a.pass_b)
    lines = [f"# Issue counters per kernel: {a.workload}", "",
             "Two counter passes of the same command, each a run of its own:", "",
             f"    {a.command}", "",
             "Per-dispatch averages (see jagged_attention_amd/counters.py for the formulas: one "
             "XCD's cycles are GRBM_GUI_ACTIVE / 8; MFMA busy over 1024 SIMDs; LDS over 256 CUs; "
             "waiting = SQ_WAIT_ANY / SQ_WAVE_CYCLES).", "",
             "| Kernel | Dispatches | Cycles (one XCD) | Waves | MFMA busy | "
             "LDS active | LDS conflict stalls | VALU instr. per MFMA | Waves waiting |",
             "|---|---|---|---|---|---|---|---|---|"]
    for n, r in rows.items():
        vpm = f"{r['valu_per_mfma']:.1f}" if r["valu_per_mfma"] else "-"
        lines.append(f"| {n} | {r['dispatches']} | {r['cycles']:,.0f} | {r['waves']:.0f} | "
                     f"{100 * r['mfma_busy']:.1f}% | {100 * r['lds_active']:.1f}% | "
                     f"{100 * r['lds_conflict']:.1f}% | {vpm} | {100 * r['waiting']:.1f}% |")
    path = os.path.join(a.out, f"{file_tag(a.workload)}_utilisation.md")
    with open(path, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


if __name__ == "__main__":
    main()
