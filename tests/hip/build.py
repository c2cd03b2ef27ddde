"""Build the tests' lane-layout probe library (tests/hip/liblane_probe.so) and the
hardware-probe program (tests/hip/hw_probe) for gfx950.

Usage: python tests/hip/build.py   (also run by the repository's build entry point)
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))
from structured_attention_video_amd.build import ARCH, FLAGS, hipcc  # noqa: E402

SRC = os.path.join(HERE, "lane_probe.hip")
OUT = os.path.join(HERE, "liblane_probe.so")
PROBE_SRC = os.path.join(HERE, "hw_probe.hip")
PROBE_OUT = os.path.join(HERE, "hw_probe")


def _hipcc(args, out):
    tmp = out + ".tmp"
    cmd = [hipcc(), *FLAGS, *args, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stderr}")
    os.replace(tmp, out)


def build(verbose: bool = True) -> str:
    """The lane-layout probe library and the hardware-probe program."""
    _hipcc(["-shared", SRC], OUT)
    _hipcc([PROBE_SRC], PROBE_OUT)
    if verbose:
        print(f"built {OUT} and {PROBE_OUT} ({ARCH})")
    return OUT


if __name__ == "__main__":
    build()
