import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


# MONARCH_HOSTSAN=1 (set only by test_abi_hostsan.py for its child run, which
# also preloads the ASan runtime): load the host-sanitizer build of the library
# instead of the in-tree one
HOSTSAN = os.environ.get("MONARCH_HOSTSAN") == "1"


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: large CPU oracle runs")
    if HOSTSAN:
        from structured_attention_video_amd import _lib, build
        _lib.LIB_PATH = build.SAN_OUT


def pytest_sessionfinish(session, exitstatus):
    if HOSTSAN:
        from structured_attention_video_amd import build
        mapped = any(build.SAN_OUT in line for line in open("/proc/self/maps"))
        print(f"\nhostsan library mapped: {mapped}", flush=True)


def pytest_collection_modifyitems(config, items):
    try:
        import torch
        have_gpu = torch.cuda.is_available()
    except Exception:  # pragma: no cover
        have_gpu = False
    if have_gpu:
        return
    skip = pytest.mark.skip(reason="no GPU visible")
    for item in items:
        if "gpu" in item.keywords:
            item.add_marker(skip)
