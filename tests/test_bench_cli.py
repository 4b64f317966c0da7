"""bench.py's command line on the CPU: more than one GPU is refused before anything runs."""

from __future__ import annotations

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_refuses_more_than_one_gpu():
    run = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], cwd=ROOT,
                         capture_output=True, text=True, timeout=120)
    assert run.returncode == 2
    assert "one GPU" in run.stderr


def test_bench_refuses_a_distributed_launch():
    env = dict(os.environ, WORLD_SIZE="4")
    run = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")], cwd=ROOT, env=env,
                         capture_output=True, text=True, timeout=120)
    assert run.returncode == 2
    assert "one GPU" in run.stderr
