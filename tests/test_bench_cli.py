"""bench.py's command-line contract on the CPU: a request for more than one GPU
is refused with a one-line JSON message and a non-zero status before any GPU
work (this build runs on one GPU; the multi-GPU design is documentation only).
"""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2", "--steps", "1",
                        "--warmup", "0"], capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert p.returncode == 2
    line = json.loads(p.stdout.strip().splitlines()[-1])
    assert line["n_gpus"] == 2
    assert "one GPU" in line["error"]
