"""The hardware probes (tests/hip/hw_probe.hip) run to completion on the GPU.

They print the MFMA issue interval, LDS read bandwidth and VALU/MFMA co-issue
figures that the flash kernel's design rests on; this test checks that every
probe ran and that the figures are physically plausible (the design's own
numbers come from the same program, with the command that ran it).
"""
import os
import re
import subprocess

import pytest

from gpu_util import say

pytestmark = pytest.mark.gpu
PROBE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "hip", "hw_probe")


def test_hw_probes_run():
    if not os.path.exists(PROBE):
        pytest.fail(f"{PROBE} is not built (python tests/hip/build.py)")
    say("hardware probes")
    r = subprocess.run([PROBE], capture_output=True, text=True, timeout=120)
    say(r.stdout)
    assert r.returncode == 0, r.stdout + r.stderr
    out = r.stdout
    assert "probes done (status 0)" in out
    per_mfma = [float(x) for x in re.findall(r"([\d.]+) memtime/MFMA", out)]
    assert len(per_mfma) == 6 and all(8.0 <= x <= 128.0 for x in per_mfma), per_mfma
    lds = [float(x) for x in re.findall(r"LDS (\d+) B/clk/CU", out)]
    assert len(lds) == 10 and all(16.0 <= x <= 512.0 for x in lds), lds
    assert len(re.findall(r"cycles per MFMA step per wave", out)) == 3
