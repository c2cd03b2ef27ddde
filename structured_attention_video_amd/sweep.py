"""Alignment / block-size / tile sweep: the error of Monarch attention against
dense attention on synthetic inputs with axis structure, and its time.

The MonarchRT pages claim that blocks aligned with the video axes keep the
separable positional part of attention exactly while misaligned blocks lose it
(gist.science explainer, Methodology A), and that restricting stage 2 to tiles
of frames keeps most of the quality for long videos (same page, Methodology B).
This sweep measures both on seeded synthetic inputs: for each input family,
each block size (frame- or row-aligned, or the divisor of N nearest to a frame
or a row that straddles rows) and each tile count, it runs the library's
forward and the library's dense kernel on the same tensors and reports the
relative L2 distance between the two outputs and the forward's device time
per call. Everything runs through the HIP library; this module only picks the
cases, draws inputs and compares outputs.

    python -m structured_attention_video_amd.sweep [--grid T H W] [--heads 12] [--d 128]
"""
from __future__ import annotations

import argparse
import json
import math
import statistics
from typing import Callable, List, Sequence, Tuple

import torch

import datagen

from .attention import MonarchPlan

# input families: name -> (grid, heads, d) -> Q, K, V (CPU, bf16)
FAMILIES: List[Tuple[str, Callable]] = [
    ("separable", lambda g, hh, d: datagen.noisy_separable_qkv(1, hh, g, d, 3000, 0.0)),
    ("separable+noise0.5", lambda g, hh, d: datagen.noisy_separable_qkv(1, hh, g, d, 3000, 0.5)),
    ("pe0.5", lambda g, hh, d: datagen.qkv(1, hh, g, d, (1000, 1001, 1002), pe_scale=0.5)),
    ("iid", lambda g, hh, d: datagen.iid_qkv(1, hh, g[0] * g[1] * g[2], d, (0, 1, 2), torch.bfloat16)),
]


def divisors(n: int) -> List[int]:
    small = [i for i in range(1, int(math.isqrt(n)) + 1) if n % i == 0]
    return sorted(set(small + [n // i for i in small]))


def block_cases(grid: Sequence[int]) -> List[Tuple[str, str, int, int]]:
    """(label, alignment, custom b, b): frame, row, and for each of those the
    divisor of N closest to it (in ratio) whose blocks straddle rows (b is
    neither a multiple nor a divisor of W)."""
    T, H, W = (int(x) for x in grid)
    N = T * H * W
    cases = [("frame", "frame", 0, H * W), ("row", "row", 0, W)]
    straddle = [b for b in divisors(N) if 1 < b < N and b % W and W % b]
    seen = {H * W, W}
    for label, target in (("misaligned~frame", H * W), ("misaligned~row", W)):
        if not straddle:
            break
        b = min(straddle, key=lambda x: (abs(math.log(x / target)), x))
        if b not in seen:
            cases.append((label, "custom", b, b))
            seen.add(b)
    return cases


def tile_counts(T: int) -> List[int]:
    """Frame-aligned tile counts U (tiles of T/U frames): the divisors of T."""
    return divisors(int(T))


def rel_l2(x: torch.Tensor, ref: torch.Tensor) -> float:
    d = (x.float() - ref.float()).norm()
    return float(d / ref.float().norm())


def _time(fn, reps: int) -> float:
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    fn()
    torch.cuda.synchronize()
    for a, b in ev:
        a.record()
        fn()
        b.record()
    torch.cuda.synchronize()
    return statistics.median(a.elapsed_time(b) for a, b in ev)


def sweep(grid: Sequence[int], heads: int = 2, d: int = 128, families=None, reps: int = 5,
          device: str = "cuda", tiles: bool = True) -> List[dict]:
    T, H, W = (int(x) for x in grid)
    N = T * H * W
    rows = []
    for fname, make in (families or FAMILIES):
        q, k, v = (x.to(device) for x in make((T, H, W), heads, d))
        dense = MonarchPlan(1, heads, d, (T, H, W), align="dense")
        od = dense.forward(q, k, v)
        t_dense = _time(lambda: dense.forward(q, k, v, out=od), reps)
        dense.close()
        cases = [(label, align, cb, b, 0) for label, align, cb, b in block_cases((T, H, W))]
        if tiles:
            cases += [(f"frame, {U} tiles", "frame", 0, H * W, N // U) for U in tile_counts(T) if U > 1]
        for label, align, cb, b, tau in cases:
            plan = MonarchPlan(1, heads, d, (T, H, W), align=align, custom_b=cb, tile_tokens=tau or None,
                               allow_unaligned=(align == "custom"))
            ws = plan.new_workspace(q.device)
            o = plan.forward(q, k, v, workspace=ws)
            ms = _time(lambda: plan.forward(q, k, v, out=o, workspace=ws), reps)
            info = plan.info
            rows.append({"family": fname, "case": label, "b": b, "tile_tokens": tau or N,
                         "tiles": N // (tau or N), "m_tau": info["m_tau"],
                         "density": round((info["b"] + info["m_tau"]) / N, 5),
                         "rel_l2_vs_dense": rel_l2(o, od), "ms_per_call": round(ms, 4),
                         "dense_ms_per_call": round(t_dense, 4)})
            plan.close()
            del ws, o
        del q, k, v, od
    return rows


def main(argv=None) -> None:
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--grid", type=int, nargs=3, default=[21, 30, 52])
    ap.add_argument("--heads", type=int, default=12)
    ap.add_argument("--d", type=int, default=128)
    ap.add_argument("--reps", type=int, default=10)
    args = ap.parse_args(argv)
    if not torch.cuda.is_available():
        raise SystemExit("the sweep runs the HIP library: no GPU is visible")
    rows = sweep(args.grid, args.heads, args.d, reps=args.reps)
    for r in rows:
        print(json.dumps(r))


if __name__ == "__main__":
    main()
