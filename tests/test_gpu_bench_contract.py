"""The bench line's contract, on the GPU: one short `bench.py` run at the default
workload (the 21x30x52-token, 12-head, d=128 bf16 frame layout) prints one JSON
line with the throughput fields, the roofline of the dominant kernel
(algorithmic FLOPs per launch over the launch's measured time, against the
2.5 PFLOP/s bf16 MFMA peak) and the oracle's CPU timing beside it, and its own
parity check against the oracle passes.
"""
import json
import os
import subprocess
import sys

import pytest

from gpu_util import say

pytestmark = pytest.mark.gpu
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_line_fields():
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--steps", "3", "--warmup", "1"],
                       capture_output=True, text=True, timeout=600, cwd=ROOT)
    assert p.returncode == 0, p.stderr[-2000:]
    lines = [ln for ln in p.stdout.splitlines() if ln.strip().startswith("{")]
    assert len(lines) == 1, p.stdout[-2000:]
    d = json.loads(lines[0])
    say(f"  value {d['value']} {d['unit']}, frac {d['roofline']['frac']}, traffic {d['roofline']['traffic']}")
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better",
                "scaling", "vs_baseline", "dtype", "data", "config", "roofline", "cpu_baseline"):
        assert key in d, key
    assert d["n_gpus"] == 1 and d["steps"] == 3 and d["warmup"] == 1
    assert d["higher_is_better"] is True and d["dtype"] == "bf16"
    assert d["config"]["workload"] == "frame_bf16" and d["config"]["grid"] == [21, 30, 52]
    assert d["value"] > 0 and d["ms_per_step"] > 0
    # throughput = the forward's FLOPs (both stages) over the measured time per step
    assert abs(d["value"] - d["flops_per_call"] / (d["ms_per_step"] * 1e-3) / 1e12) <= 0.01 * d["value"]
    r = d["roofline"]
    for key in ("bound", "achieved", "peak", "unit", "frac", "traffic"):
        assert key in r, key
    assert r["bound"] == "mfma" and r["unit"] == "TFLOP/s" and r["peak"] == 2500.0
    assert abs(r["frac"] - r["achieved"] / r["peak"]) < 1e-3
    assert r["traffic"] is None or r["traffic"] > 0
    c = d["cpu_baseline"]
    assert c["kind"] == "oracle" and c["value"] > 0 and c["cores"] >= 1 and c["sample"]
    pv = d["parity_vs_oracle"]
    assert pv["rel_l2"] <= 1e-2 and pv["max_abs"] <= 3e-2
