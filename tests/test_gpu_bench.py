"""bench.py end to end on the smallest workload (fp32 token rows, head_dim 64): one JSON line
with the fields its contract names, run as a child process the way it is launched."""

from __future__ import annotations

import json
import os
import subprocess
import sys

import pytest

import gpu_util as G

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(autouse=True)
def _gpu():
    G.need_gpu()


def test_bench_tiny_prints_one_contract_line():
    cmd = [sys.executable, os.path.join(ROOT, "bench.py"), "--workload", "tiny", "--steps", "3", "--warmup", "1",
           "--no-cpu-baseline"]
    run = subprocess.run(cmd, cwd=ROOT, capture_output=True, text=True, timeout=240)
    assert run.returncode == 0, run.stderr[-2000:]
    lines = [json.loads(line) for line in run.stdout.splitlines() if line.startswith("{")]
    assert len(lines) == 1, run.stdout[-2000:]
    rec = lines[0]
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better",
                "scaling", "vs_baseline", "dtype", "data", "config", "roofline"):
        assert key in rec, key
    assert rec["n_gpus"] == 1 and rec["steps"] == 3 and rec["warmup"] == 1
    assert rec["value"] > 0 and rec["ms_per_step"] > 0
    assert rec["config"]["workload"].startswith("tiny")
    roof = rec["roofline"]
    for key in ("bound", "achieved", "peak", "unit", "frac", "traffic"):
        assert key in roof, key
    assert roof["bound"] == "mfma" and 0 < roof["frac"] < 1
    assert roof["kernel"].startswith("attention_kernel<64, false>") or roof["kernel"].startswith(
        "attention_split_kernel<64, false>")
    # fp32 token rows: the standalone gather (bf16 rows only) is left out of the HBM steps
    assert "a4_gather" not in rec["hbm_kernels"] and "a1_score" in rec["hbm_kernels"]

