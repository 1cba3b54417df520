"""bench.py's command-line contract, on the CPU: it runs on one GPU only and
says so for --gpus N > 1, and it refuses conflicting modes; both exits happen
before any GPU work."""

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                          timeout=120)


def test_more_than_one_gpu_is_refused_with_a_message():
    r = run("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


def test_conflicting_modes_are_refused():
    r = run("--stats", "--lse-in")
    assert r.returncode == 2
    assert "separate modes" in r.stderr
