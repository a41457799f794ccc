"""bench.py's command-line contract that holds without a GPU.

The library and every figure bench.py reports are one GPU's, so a request for
more GPUs is refused with a message before anything touches a device.
"""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                          timeout=120, cwd=ROOT)


def test_more_than_one_gpu_is_refused_with_a_message():
    r = _run("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""  # no JSON line for a run that did not happen


def test_unknown_workload_is_rejected():
    r = _run("--workload", "no_such_workload")
    assert r.returncode != 0
    assert "invalid choice" in r.stderr
