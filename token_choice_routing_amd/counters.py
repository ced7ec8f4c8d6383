"""Per-kernel medians of rocprofv3 counters, one markdown table.

Usage:

    python -m token_choice_routing_amd.counters TITLE COMMAND KERNEL_PREFIX CSV [CSV ...]

Each CSV is the ``*_counter_collection.csv`` of one ``rocprofv3 --pmc <counters>``
run (one run per counter set: the hardware collects a limited number per block at
once). For the dispatches whose kernel name starts with KERNEL_PREFIX, every
counter's value per dispatch (summed over the rows rocprofv3 writes for it) and its
median over the dispatches are printed, plus ratios of counters in the same units
when both are present: SQ_WAIT_INST_ANY and SQ_ACTIVE_INST_ANY over SQ_WAVE_CYCLES
(the share of wave time stalled on a dependency, and issuing), and
SQ_LDS_BANK_CONFLICT over SQ_LDS_IDX_ACTIVE.
"""
import csv
import statistics
import sys


def per_dispatch(path, prefix):
    out = {}
    with open(path, newline="") as f:
        for r in csv.DictReader(f):
            if not r["Kernel_Name"].startswith(prefix):
                continue
            d = out.setdefault(r["Counter_Name"], {})
            d[r["Dispatch_Id"]] = d.get(r["Dispatch_Id"], 0.0) + float(r["Counter_Value"])
    return out


def main(argv):
    if len(argv) < 5:
        print(__doc__)
        return 2
    title, cmd, prefix, csvs = argv[1], argv[2], argv[3], argv[4:]
    med, n = {}, {}
    for path in csvs:
        for c, d in per_dispatch(path, prefix).items():
            med[c] = statistics.median(d.values())
            n[c] = len(d)
    print(f"# {title}\n\nCommands (each counter set its own run, from /tmp with TMPDIR=/tmp on one MI355X):\n")
    print(f"```\n{cmd}\npython -m token_choice_routing_amd.counters <title> <command> '{prefix}' <csv> ...\n```\n")
    print(f"Kernel: `{prefix}`. Values are per dispatch (summed over the chip), medians over dispatches.\n")
    print("| counter | median per dispatch | dispatches |\n|---|---|---|")
    for c in sorted(med):
        print(f"| {c} | {med[c]:.4e} | {n[c]} |")
    print()
    ratios = []
    if "SQ_WAIT_INST_ANY" in med and "SQ_WAVE_CYCLES" in med:
        ratios.append(("waves stalled on a dependency (SQ_WAIT_INST_ANY / SQ_WAVE_CYCLES)",
                       med["SQ_WAIT_INST_ANY"] / med["SQ_WAVE_CYCLES"]))
    if "SQ_ACTIVE_INST_ANY" in med and "SQ_WAVE_CYCLES" in med:
        ratios.append(("waves issuing (SQ_ACTIVE_INST_ANY / SQ_WAVE_CYCLES)",
                       med["SQ_ACTIVE_INST_ANY"] / med["SQ_WAVE_CYCLES"]))
    if "SQ_LDS_BANK_CONFLICT" in med and med.get("SQ_LDS_IDX_ACTIVE"):
        ratios.append(("LDS bank-conflict cycles / LDS active cycles",
                       med["SQ_LDS_BANK_CONFLICT"] / med["SQ_LDS_IDX_ACTIVE"]))
    if ratios:
        print("| ratio | value |\n|---|---|")
        for name, v in ratios:
            print(f"| {name} | {v:.3f} |")
    return 0


if __name__ == "__main__":
    sys.exit(main(sys.argv))
