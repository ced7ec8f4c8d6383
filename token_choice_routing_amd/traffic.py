"""HBM traffic per kernel launch from two rocprofv3 counter passes.

Usage (after the two passes described in the summary this writes):

    python -m token_choice_routing_amd.traffic FETCH_CSV WRITE_CSV WORKLOAD [OUT_DIR]

FETCH_CSV / WRITE_CSV are the ``*_counter_collection.csv`` files of a
``rocprofv3 --pmc FETCH_SIZE`` run and a ``rocprofv3 --pmc WRITE_SIZE`` run of
``bench.py --copy-ref`` (each counter in its own run). Both counters are KiB per
dispatch. They are scaled by what the same counter reads for the reference copy
kernel (``__amd_rocclr_copyBuffer``, 256 MiB read and 256 MiB written), so the
result is bytes moved between the last-level cache and HBM per launch. The
median over a kernel's dispatches is reported.

Writes ``traffic.json`` (read by bench.py as the roofline ``traffic`` field) and a
markdown summary into OUT_DIR (default: profiles/ at the repository root).
"""
import csv
import json
import os
import statistics
import sys

COPY_KERNEL = "__amd_rocclr_copyBuffer"
COPY_BYTES = 256 << 20

# bench.py kernel-table names -> kernel-name prefixes (GEMM template arguments: mode
# 0 gate/up, 2 half-precision down; role 0 standalone grouped, 1 standalone single
# segment, 2 the layer's launches); either GEMM kernel may run a launch
def _gemm(mode, role):
    return (f"void moe::grouped_gemm_bf16_kernel<{mode}, {role},", f"void moe::grouped_gemm_pp_kernel<{mode}, {role}>")


BENCH_KERNELS = {
    "gate_up_layer": _gemm(0, 2),
    "down_layer": _gemm(2, 2),
    "down_combine_layer": ("void moe::grouped_gemm_pp_kernel<3, 2>",),
    "gemm_gate_up": _gemm(0, 0),
    "gemm_down": _gemm(2, 0),
    "shared_gate_up": _gemm(0, 1),
    "shared_down": _gemm(2, 1),
    "route": ("void moe::route_tile_kernel<false,",),
    "layer_route": ("void moe::route_tile_kernel<true,",),
    "gather": ("moe::gather_rows_kernel",),
    "combine": ("void moe::combine_kernel<",),
}


def read_counter(path, counter):
    """{kernel name: [KiB per dispatch, ...]} for one counter."""
    out = {}
    with open(path, newline="") as f:
        for row in csv.DictReader(f):
            if row.get("Counter_Name") != counter:
                continue
            out.setdefault(row["Kernel_Name"], []).append(float(row["Counter_Value"]))
    return out


def copy_scale(values, counter):
    """Reference bytes / counted bytes for the copy kernel's full-size dispatches."""
    kib = [v for v in values.get(COPY_KERNEL, []) if v * 1024 > COPY_BYTES / 8]
    if not kib:
        raise SystemExit(f"no {COPY_KERNEL} dispatch of the reference size in the {counter} pass "
                         "(run bench.py with --copy-ref)")
    return COPY_BYTES / (statistics.median(kib) * 1024)


def summarize(fetch_csv, write_csv):
    fetch = read_counter(fetch_csv, "FETCH_SIZE")
    write = read_counter(write_csv, "WRITE_SIZE")
    fs, ws = copy_scale(fetch, "FETCH_SIZE"), copy_scale(write, "WRITE_SIZE")
    rows = {}
    for name in sorted(set(fetch) | set(write)):
        f = statistics.median(fetch[name]) * 1024 * fs if name in fetch else None
        w = statistics.median(write[name]) * 1024 * ws if name in write else None
        rows[name] = {"fetch_bytes": f, "write_bytes": w,
                      "dispatches": max(len(fetch.get(name, [])), len(write.get(name, [])))}
    return rows, fs, ws


def main(argv):
    if len(argv) < 4:
        print(__doc__)
        return 2
    fetch_csv, write_csv, workload = argv[1], argv[2], argv[3]
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    out_dir = argv[4] if len(argv) > 4 else os.path.join(root, "profiles")
    rows, fs, ws = summarize(fetch_csv, write_csv)
    path = os.path.join(out_dir, "traffic.json")
    tab = json.load(open(path)) if os.path.exists(path) else {}
    for short, prefix in BENCH_KERNELS.items():
        hits = [n for n in rows if n.startswith(prefix)]
        if len(hits) != 1:
            continue
        r = rows[hits[0]]
        if r["fetch_bytes"] is None or r["write_bytes"] is None:
            continue
        tab[f"{short}@{workload}"] = {
            "kernel": hits[0].split("(")[0], "bytes_per_launch": round(r["fetch_bytes"] + r["write_bytes"]),
            "fetch_bytes": round(r["fetch_bytes"]), "write_bytes": round(r["write_bytes"]),
            "fetch_scale": round(fs, 4), "write_scale": round(ws, 4)}
    with open(path, "w") as f:
        json.dump(tab, f, indent=1, sort_keys=True)
    md = os.path.join(out_dir, f"traffic_kernels_{workload}.md")
    with open(md, "w") as f:
        f.write(f"# HBM traffic per launch, {workload}\n\n")
        f.write("Two counter passes, each its own run, from /tmp with TMPDIR=/tmp on one MI355X:\n\n```\n")
        for c in ("FETCH_SIZE", "WRITE_SIZE"):
            f.write(f"timeout -s KILL 150 rocprofv3 --pmc {c} --output-format csv -d <out> -o run -- "
                    "python3 bench.py --no-sweep --no-cpu --steps 2 --warmup 1 --kernel-iters 3 --copy-ref\n")
        f.write(f"python -m token_choice_routing_amd.traffic <fetch csv> <write csv> {workload}\n```\n\n")
        f.write(f"Counters are KiB per dispatch, scaled by the reference copy of {COPY_BYTES >> 20} MiB: "
                f"FETCH_SIZE x {fs:.4f}, WRITE_SIZE x {ws:.4f}. Median over dispatches. The bench "
                "flushes the last-level cache before each timed GEMM launch of its kernel table.\n\n")
        f.write("| kernel | dispatches | read MB | written MB |\n|---|---|---|---|\n")
        for name, r in sorted(rows.items(), key=lambda kv: -((kv[1]["fetch_bytes"] or 0) + (kv[1]["write_bytes"] or 0))):
            fb = "" if r["fetch_bytes"] is None else f"{r['fetch_bytes'] / 1e6:.2f}"
            wb = "" if r["write_bytes"] is None else f"{r['write_bytes'] / 1e6:.2f}"
            f.write(f"| `{name.split('(')[0]}` | {r['dispatches']} | {fb} | {wb} |\n")
    print(f"wrote {path} and {md}")
    return 0


if __name__ == "__main__":
    sys.exit(main(sys.argv))
