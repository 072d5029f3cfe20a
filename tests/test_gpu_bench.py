"""bench.py end to end on the small workloads (one of them ragged): it runs,
prints one JSON line with the contract's fields, and the roofline and
e2e figures are positive. The headline workload is exercised by the
benchmark run itself."""
from __future__ import annotations

import json
import os
import subprocess
import sys

import pytest
import torch

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FIELDS = ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
          "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config", "roofline",
          "cpu_baseline")


@pytest.mark.parametrize("config", [1, 2])
def test_bench_small_workloads(config):
    print(f"[test] bench.py --config {config}", flush=True)
    extra = [] if config == 1 else ["--no-prefill"]
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--config",
                          str(config), "--steps", "3", "--warmup", "1", "--no-cpu-baseline",
                          *extra], capture_output=True, text=True, timeout=240, cwd=ROOT)
    assert res.returncode == 0, res.stderr[-3000:]
    lines = [l for l in res.stdout.splitlines() if l.startswith("{")]
    assert len(lines) == 1, res.stdout[-2000:]
    d = json.loads(lines[0])
    for f in FIELDS:
        assert f in d, f
    assert d["n_gpus"] == 1 and d["steps"] == 3 and d["value"] > 0
    r = d["roofline"]
    assert r["bound"] == "hbm" and 0 < r["frac"] < 1.5
    probe = r["stream_read_probe"]
    assert probe["same_bytes"]["launch_ms"] > 0 and probe["4_gib"]["achieved"] > 0
    e2e = d["e2e"]
    pairs = e2e["per_step_event_pairs"]
    assert e2e["frac_of_peak"] > 0 and pairs["step_ms_p50"] <= pairs["step_ms_p90"]
    assert e2e["timing"]
    assert "three_launch_chain" in e2e["other_forms"]
    if config == 1:
        assert d["prefill"]["achieved_tflops"] > 0
    else:
        assert d["prefill"] is None
