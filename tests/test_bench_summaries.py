"""bench.py's profile summaries on synthetic rocprofv3 CSVs (no GPU).

The committed profiles and the bench line's roofline.traffic come from these
functions, so their arithmetic is checked here against hand-computed values:
the stage-1 kernel's mean launch time and roofline fraction from a kernel
trace, HBM bytes per launch from FETCH_SIZE / WRITE_SIZE scaled by a copy of
known size, and the digest guard on stored traffic figures.
"""
import csv
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402

FLASH = "void monarch::(anonymous namespace)::flash_kernel<128, false, false, false, false>(monarch::GroupedArgs, int, int, int)"
GROUP = "void monarch::(anonymous namespace)::group_kernel<128, 1, false>(monarch::GroupedArgs)"


def _write(path, header, rows):
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(header)
        w.writerows(rows)
    return str(path)


def _run(*args):
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                       timeout=120, cwd=ROOT)
    assert p.returncode == 0, p.stderr
    return p.stdout


def test_trace_summary_mean_and_fraction(tmp_path):
    # three stage-1 launches of 300, 310 and 320 us on the frame grid, one of another grid (a
    # different workload of the same kernel), two stage-2 launches
    rows, t = [], 0
    for name, grid, us in [(FLASH, 838656, 300), (GROUP, 1198080, 70), (FLASH, 838656, 310),
                           (FLASH, 786432, 6000), (GROUP, 1198080, 72), (FLASH, 838656, 320)]:
        rows.append([name, grid, t, t + us * 1000])
        t += us * 1000 + 5000
    path = _write(tmp_path / "trace.csv", ["Kernel_Name", "Grid_Size_X", "Start_Timestamp", "End_Timestamp"], rows)
    out = _run("--trace-summary", path, "--config", "frame_bf16")
    assert "3 launches, mean 310.0 us" in out
    flops = 4 * 12 * 32760 * 1560 * 128
    frac = flops / 310e-6 / 2.5e15
    assert f"frac {frac:.4f}" in out
    # the row layout's flash kernel is its stage 2 (m = 630 > 128)
    out = _run("--trace-summary", path, "--config", "row_bf16")
    assert "stage-2 kernel" in out


def test_traffic_summary_scales_by_the_copy(tmp_path):
    hdr = ["Kernel_Name", "Grid_Size", "Counter_Name", "Counter_Value"]
    gib_kib = (1 << 30) / 1024
    fetch = _write(tmp_path / "f.csv", hdr, [[FLASH, 838656, "FETCH_SIZE", 150000.0],
                                             [FLASH, 838656, "FETCH_SIZE", 160000.0],
                                             [GROUP, 1198080, "FETCH_SIZE", 140000.0]])
    write = _write(tmp_path / "w.csv", hdr, [[FLASH, 838656, "WRITE_SIZE", 100000.0],
                                             [GROUP, 1198080, "WRITE_SIZE", 98000.0]])
    # the copy reads and writes 1 GiB; its FETCH_SIZE reads half of that (factor 2)
    cf = _write(tmp_path / "cf.csv", hdr, [["__amd_rocclr_copyBuffer", 65536, "FETCH_SIZE", gib_kib / 2]])
    cw = _write(tmp_path / "cw.csv", hdr, [["__amd_rocclr_copyBuffer", 65536, "WRITE_SIZE", gib_kib]])
    out = _run("--traffic-summary", fetch, write, cf, cw, "--config", "frame_bf16")
    assert "FETCH_SIZE factor 2.000, WRITE_SIZE factor 1.000" in out
    want = (155000.0 * 1024 * 2) + (100000.0 * 1024 * 1)
    line = [x for x in out.splitlines() if x.startswith("hbm_bytes_per_launch:")][0]
    assert float(line.split(":")[1]) == pytest.approx(want, rel=1e-5)
    assert f"source_digest: {bench.source_digest()}" in out


def test_stored_traffic_needs_the_current_digest(tmp_path, monkeypatch):
    digest = bench.source_digest()
    assert len(digest) == 16
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "source_digest", lambda: digest)
    os.makedirs(tmp_path / "profiles")
    f = tmp_path / "profiles" / "traffic_flash_mfma_bf16_frame_bf16.txt"
    f.write_text(f"# a summary\nsource_digest: {digest}\nhbm_bytes_per_launch: 4.25e+08\n")
    assert bench.stored_traffic("flash_mfma_bf16", "frame_bf16") == pytest.approx(4.25e8)
    f.write_text("source_digest: 0000000000000000\nhbm_bytes_per_launch: 4.25e+08\n")
    assert bench.stored_traffic("flash_mfma_bf16", "frame_bf16") is None
    assert bench.stored_traffic("flash_mfma_bf16", "row_bf16") is None
