"""Per-kernel duration summary of a rocprofv3 kernel trace.

Usage:

    python -m token_choice_routing_amd.profsummary RESULTS_DB TITLE COMMAND > summary.md

RESULTS_DB is the ``*_results.db`` that ``rocprofv3 --kernel-trace --stats -d <dir>
-o run`` writes; COMMAND is the command that made it (printed into the summary).
Besides the per-kernel totals this splits every kernel's dispatches into cold ones
(the kernel dispatched right before it was the cache-flushing 512 MB sum that
bench.py issues before each timed GEMM launch of its kernel table) and warm ones
(any other predecessor), because bench.py's roofline uses the cold launches.
"""
import sqlite3
import statistics
import sys


def is_flush(name):
    """torch's reduction kernel for a float32 sum (bench.py's flush)."""
    return name.startswith("void at::native::reduce_kernel<") and "sum_functor<float" in name


def short(name):
    """Kernel name without its argument list (and without the anonymous namespace,
    whose parentheses would otherwise end the name)."""
    return name.replace("(anonymous namespace)::", "").split("(")[0]


def dispatches(db):
    """[(name, duration ns)] in start order, with a cold flag per dispatch."""
    con = sqlite3.connect(db)
    rows = con.execute("select name, start, duration from kernels order by start").fetchall()
    con.close()
    out, prev = [], ""
    for name, _start, dur in rows:
        out.append((name, dur, is_flush(prev)))
        prev = name
    return out


def summarize(db):
    per = {}
    for name, dur, cold in dispatches(db):
        e = per.setdefault(name, {"all": [], "cold": [], "warm": []})
        e["all"].append(dur)
        e["cold" if cold else "warm"].append(dur)
    return per


def fmt_avg(ns):
    return f"{statistics.mean(ns) / 1e3:.3f}" if ns else ""


def main(argv):
    if len(argv) < 4:
        print(__doc__)
        return 2
    db, title, cmd = argv[1], argv[2], argv[3]
    per = summarize(db)
    total = sum(sum(e["all"]) for e in per.values()) or 1
    print(f"# {title}\n\nCommand (run from /tmp with TMPDIR=/tmp on one MI355X):\n\n```\n{cmd}\n"
          f"python -m token_choice_routing_amd.profsummary <out>/run_results.db <title> <command>\n```\n")
    print("Cold = dispatched directly after the cache-flushing sum; warm = any other dispatch.\n")
    print("| kernel | calls | total us | average us | % | cold calls | cold avg us | warm calls | warm avg us |")
    print("|---|---|---|---|---|---|---|---|---|")
    for name, e in sorted(per.items(), key=lambda kv: -sum(kv[1]["all"])):
        s = sum(e["all"])
        print(f"| `{short(name)}` | {len(e['all'])} | {s / 1e3:.1f} | {fmt_avg(e['all'])} | "
              f"{100 * s / total:.1f} | {len(e['cold'])} | {fmt_avg(e['cold'])} | "
              f"{len(e['warm'])} | {fmt_avg(e['warm'])} |")
    return 0


if __name__ == "__main__":
    sys.exit(main(sys.argv))
