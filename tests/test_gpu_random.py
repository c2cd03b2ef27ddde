"""Seeded random shapes through the HIP library against the fp64 oracle.

Each case draws a grid, head dim, dtype, batch, heads and an alignment (frame,
row, dense, token, a misaligned custom block size, or frame-aligned tiles),
runs the forward into a guard-banded output, and compares it with the oracle
element by element at the usual tolerance (bf16 rel-L2 <= 1e-2, max-abs <=
3e-2; fp32 <= 1e-5). Every bf16 case with a backward also checks the
gradients against the oracle backward. The cases are fixed by the seed, so a
failure names a reproducible shape.
"""
import numpy as np
import pytest
import torch

import datagen
import oracle
from gpu_util import assert_close, say, to_np
from structured_attention_video_amd import MonarchPlan
from test_gpu_backward import check as check_grad
from test_gpu_parity import run

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def divisors(n):
    return [i for i in range(1, n + 1) if n % i == 0]


def draw_cases(seed=20260, n=24):
    rng = np.random.default_rng(seed)
    cases = []
    while len(cases) < n:
        T, H, W = int(rng.integers(1, 7)), int(rng.integers(1, 9)), int(rng.integers(1, 41))
        N = T * H * W
        if N < 2 or N > 1500:
            continue
        d = int(rng.choice([64, 128]))
        dtype = "fp32" if rng.random() < 0.2 else "bf16"
        align = str(rng.choice(["frame", "row", "dense", "token", "custom", "tiled"]))
        cb, tile = 0, 0
        if align == "dense" and N > 600:
            align = "frame"
        if align == "custom":
            cands = [b for b in divisors(N) if b not in (1, W, H * W, N)]
            if not cands:
                continue
            cb = int(rng.choice(cands))
        if align == "tiled":
            if T < 2:
                continue
            align = "frame"
            tile = H * W * int(rng.choice([k for k in divisors(T) if k < T]))
        batch, heads = int(rng.integers(1, 3)), int(rng.integers(1, 4))
        cases.append(((T, H, W), d, dtype, align, cb, tile, batch, heads, int(rng.integers(0, 1 << 30))))
    return cases


CASES = draw_cases()


@pytest.mark.parametrize("case", CASES, ids=[f"{c[0][0]}x{c[0][1]}x{c[0][2]}-d{c[1]}-{c[2]}-{c[3]}"
                                              f"-b{c[4]}-t{c[5]}-B{c[6]}H{c[7]}" for c in CASES])
def test_random_shape(case):
    grid, d, dtype, align, cb, tile, batch, heads, seed = case
    dt = datagen.torch_dtype(dtype)
    q, k, v = datagen.qkv(batch, heads, grid, d, (seed, seed + 1, seed + 2), dtype=dt)
    b = oracle.block_size(grid, align, cb)
    got = run(q, k, v, grid, align, tile, cb, allow_unaligned=(align == "custom"))
    assert_close(to_np(got), oracle.monarch_forward(q, k, v, b, tile or None), dt,
                 f"{grid} d{d} {dtype} {align} b={b} t{tile}")
    plan = MonarchPlan(batch, heads, d, grid, align=align, tile_tokens=tile, custom_b=cb, dtype=dt,
                       allow_unaligned=(align == "custom"))
    if dtype != "bf16" or not plan.backward_workspace_bytes:
        return
    g = datagen.qkv(batch, heads, grid, d, (seed + 3, seed + 4, seed + 5), dtype=dt)[0]
    qd, kd, vd, gd = (x.to(DEV) for x in (q, k, v, g))
    o = plan.forward(qd, kd, vd)
    grads = plan.backward(qd, kd, vd, o, gd)
    torch.cuda.synchronize()
    want = oracle.monarch_backward(q, k, v, g, b, tile or None)
    for name, x, y in zip(("dQ", "dK", "dV"), grads, want):
        check_grad(to_np(x), y, f"{grid} {align} b={b} t{tile} {name}")
    say(f"  backward ok")
