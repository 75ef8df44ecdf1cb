"""bench.py prints one JSON line with the fields its readers rely on.

A short run on the V2-Lite workload (a child process, as the bench is run):
the metric and unit, the step statistics, the roofline object of the decode
kernel and the configuration; the CPU baseline is skipped here.
"""
import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_json_line(gpu_lib):
    from gpu_util import say
    say("[bench.py json line]")
    cmd = [sys.executable, os.path.join(ROOT, "bench.py"), "--workload", "v2lite_b32_l4096", "--steps", "3",
           "--warmup", "1", "--settle-ms", "10", "--no-cpu-baseline"]
    r = subprocess.run(cmd, cwd=ROOT, capture_output=True, text=True, timeout=140)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [ln for ln in r.stdout.splitlines() if ln.strip()]
    assert len(lines) == 1, r.stdout
    b = json.loads(lines[0])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better",
                "scaling", "vs_baseline", "dtype", "data", "config", "roofline"):
        assert key in b, key
    assert b["n_gpus"] == 1 and b["steps"] == 3 and b["warmup"] == 1
    assert b["unit"] == "TFLOP/s" and b["higher_is_better"] is True and b["dtype"] == "bf16"
    assert b["value"] > 0 and b["ms_per_step"] > 0
    assert b["step_ms_p10"] <= b["step_ms_median"] <= b["step_ms_p90"]
    assert b["config"]["workload"] == "v2lite_b32_l4096"
    rf = b["roofline"]
    assert rf["bound"] == "hbm" and rf["peak"] == 8000.0 and rf["unit"] == "GB/s"
    assert 0 < rf["frac"] < 1 and abs(rf["frac"] - rf["achieved"] / rf["peak"]) < 1e-3


def test_bench_oracle_check(gpu_lib):
    """With the CPU baseline on, the bench compares the timed step's output
    with the float64 oracle on the sequences the baseline samples."""
    from gpu_util import MAX_ABS, REL_L2, say
    say("[bench.py oracle check]")
    cmd = [sys.executable, os.path.join(ROOT, "bench.py"), "--workload", "v2lite_b32_l4096", "--steps", "2",
           "--warmup", "1", "--settle-ms", "10"]
    r = subprocess.run(cmd, cwd=ROOT, capture_output=True, text=True, timeout=110)
    assert r.returncode == 0, r.stderr[-2000:]
    b = json.loads([ln for ln in r.stdout.splitlines() if ln.strip()][-1])
    cb = b["cpu_baseline"]
    assert cb["kind"] == "oracle" and cb["value"] > 0
    oc = cb["oracle_check"]
    say(f"  {oc['sequences']} sequences: out rel L2 {oc['out_rel_l2']:.3e}, "
        f"max-abs ratio {oc['out_max_abs_ratio']:.3e}")
    assert oc["sequences"] >= 1
    assert oc["out_rel_l2"] <= REL_L2 and oc["out_max_abs_ratio"] <= MAX_ABS
