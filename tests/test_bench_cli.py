"""bench.py's command-line contract, checked without a GPU: it measures one GPU and says so
when asked for more, and it rejects option combinations it does not support (before any
device work)."""

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, timeout=300, cwd=ROOT)


def test_more_than_one_gpu_exits_with_a_message():
    r = _run("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_duplicate_prefix_needs_the_prefix_shared_workload():
    r = _run("--workload", "llama2_7b", "--duplicate-prefix")
    assert r.returncode == 2
    assert "--duplicate-prefix" in r.stderr
