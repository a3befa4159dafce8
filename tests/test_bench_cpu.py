"""bench.py's contract checks that need no GPU: it measures one GPU only, so
--gpus above 1 exits with a message (before touching a device), and its
argument parser knows the documented options."""

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], cwd=ROOT,
                          capture_output=True, text=True, timeout=120)


def test_more_than_one_gpu_exits_with_a_message():
    p = _run("--gpus", "2")
    assert p.returncode == 2
    assert "one GPU" in p.stderr
    assert p.stdout == ""


def test_help_lists_the_options():
    p = _run("--help")
    assert p.returncode == 0
    for opt in ("--gpus", "--steps", "--warmup", "--counters-probe", "--mlp-probe", "--no-cpu-baseline"):
        assert opt in p.stdout, opt
