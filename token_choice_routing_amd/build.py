"""Builds libmoe_mi355x.so for gfx950 with hipcc, in-tree.

    python -m token_choice_routing_amd.build

Every call compiles all sources (one hipcc process per file, in parallel) and
links the shared library next to this file.
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libmoe_mi355x.so")
SOURCES = ["api.hip", "route.hip", "permute.hip", "ffn.hip", "combine.hip", "aux.hip", "backward.hip", "validate.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-result",
    # packed float32 VALU ops stay off: only ordinary float code is emitted
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    return r.returncode, out


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    objs, cmds = [], []
    for src in SOURCES:
        obj = os.path.join(BUILD, src.replace(".hip", ".o"))
        objs.append(obj)
        cmds.append([HIPCC, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj])
    with ThreadPoolExecutor(max_workers=min(len(cmds), os.cpu_count() or 4, 8)) as ex:
        results = list(ex.map(_run, cmds))
    for cmd, (rc, out) in zip(cmds, results):
        if out.strip() and (verbose or rc):
            print(out, file=sys.stderr)
        if rc:
            raise RuntimeError(f"hipcc failed: {' '.join(cmd)}")
    tmp = LIB + ".tmp"
    rc, out = _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs])
    if rc:
        print(out, file=sys.stderr)
        raise RuntimeError("link failed")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
