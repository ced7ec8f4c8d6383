"""bench.py's command line without a GPU: more than one GPU is refused with a message
(the path is built and measured for one GPU), and an unknown workload is refused."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], cwd=ROOT,
                          stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True, timeout=300)


def test_more_than_one_gpu_is_refused():
    r = _run("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout == ""


def test_unknown_workload_is_refused():
    r = _run("--workload", "no_such_workload")
    assert r.returncode == 2
    assert "unknown workload" in r.stderr
