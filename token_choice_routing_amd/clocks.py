"""Shader clock and MFMA busy fraction per kernel launch from one rocprofv3 run.

Usage:

    python -m token_choice_routing_amd.clocks COUNTER_CSV KERNEL_TRACE_CSV TITLE COMMAND

from one ``rocprofv3 --kernel-trace --pmc GRBM_GUI_ACTIVE GRBM_COUNT
SQ_BUSY_CU_CYCLES SQ_VALU_MFMA_BUSY_CYCLES`` run of ``bench.py``. GRBM_COUNT counts
shader clocks on each of the 8 XCDs, so GRBM_COUNT / 8 over the dispatch's
duration (kernel trace) is the clock the launch ran at; SQ_VALU_MFMA_BUSY_CYCLES
over (SIMDs x clocks) is the fraction of SIMD cycles the matrix cores were busy.
Prints a markdown summary (median over each kernel's dispatches).
"""
import csv
import statistics
import sys

from token_choice_routing_amd.traffic import BENCH_KERNELS

XCDS = 8
SIMDS = 256 * 4  # MI355X: 256 CUs of 4 SIMDs


def per_dispatch(counter_csv, trace_csv):
    dur = {}
    with open(trace_csv, newline="") as f:
        for r in csv.DictReader(f):
            dur[r["Dispatch_Id"]] = (r["Kernel_Name"], int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    vals = {}
    with open(counter_csv, newline="") as f:
        for r in csv.DictReader(f):
            d = vals.setdefault(r["Dispatch_Id"], {})
            d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    out = {}
    for k, v in vals.items():
        if k not in dur or "GRBM_COUNT" not in v:
            continue
        name, ns = dur[k]
        clocks = v["GRBM_COUNT"] / XCDS
        out.setdefault(name, []).append({
            "us": ns / 1e3, "ghz": clocks / ns if ns else 0.0,
            "mfma_busy": v.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0) / (SIMDS * clocks) if clocks else 0.0})
    return out


def main(argv):
    if len(argv) < 5:
        print(__doc__)
        return 2
    rows = per_dispatch(argv[1], argv[2])
    print(f"# {argv[3]}\n\nCommand (run from /tmp with TMPDIR=/tmp on one MI355X):\n\n```\n{argv[4]}\n"
          "python -m token_choice_routing_amd.clocks <counter csv> <kernel trace csv> <title> <command>\n```\n")
    print("Clock = GRBM_COUNT / 8 XCDs over the dispatch's duration; MFMA busy = "
          "SQ_VALU_MFMA_BUSY_CYCLES / (1024 SIMDs x clocks). Medians over dispatches. The counters "
          "cover a window somewhat wider than the kernel, so a short dispatch (tens of us) shows "
          "a clock above the 2.4 GHz maximum; only the long ones read true.\n")
    print("| kernel | bench name | dispatches | us | clock GHz | MFMA busy |\n|---|---|---|---|---|---|")
    for short, prefix in BENCH_KERNELS.items():
        for name, ds in rows.items():
            if name.startswith(prefix):
                med = lambda key: statistics.median(x[key] for x in ds)  # noqa: E731
                print(f"| `{name.split('(')[0]}` | {short} | {len(ds)} | {med('us'):.1f} | "
                      f"{med('ghz'):.2f} | {med('mfma_busy'):.3f} |")
    return 0


if __name__ == "__main__":
    sys.exit(main(sys.argv))
