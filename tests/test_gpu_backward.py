"""GPU parity of the backward pass (dQ, dK, dV through both stages) against
the fp64 backward oracle, which is itself pinned by finite differences and
autograd (test_oracle_backward_pins.py).

Tolerance (bf16 inputs; Y, dY, P and dS enter matrix products in bf16, all
sums in fp32): per gradient tensor, rel-L2 <= 1e-2 (norms below 1e-3 per
element count as 1e-3) and max-abs <= 3e-2 times max(1, max |reference|) -
the forward's bar, relative to the gradient's scale.
"""
import numpy as np
import pytest
import torch

import datagen
import oracle
from structured_attention_video_amd import MonarchPlan
from gpu_util import say, to_np

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
BF16 = torch.bfloat16


def check(got, want, what):
    got, want = np.asarray(got, np.float64), np.asarray(want, np.float64)
    # (a gradient that is exactly zero, e.g. dQ with a single key, is measured
    # against an absolute floor instead of its own norm)
    rel = np.linalg.norm(got - want) / max(np.linalg.norm(want), 1e-3 * np.sqrt(want.size))
    mx = np.abs(got - want).max()
    bound = 3e-2 * max(1.0, np.abs(want).max())
    say(f"  {what}: rel-L2 {rel:.2e}, max-abs {mx:.2e} (bound {bound:.2e})")
    assert np.isfinite(got).all(), what
    assert rel <= 1e-2 and mx <= bound, f"{what}: rel-L2 {rel:.3e} max-abs {mx:.3e}"


def grads(q, k, v, g, grid, align="frame", tile=0, custom_b=0):
    B, Hh, N, d = q.shape
    plan = MonarchPlan(B, Hh, d, grid, align=align, tile_tokens=tile, custom_b=custom_b, dtype=q.dtype,
                       allow_unaligned=(align == "custom"))
    say(f"  plan b={plan.info['b']} m_tau={plan.info['m_tau']} ws={plan.backward_workspace_bytes}")
    qd, kd, vd, gd = (x.to(DEV) for x in (q, k, v, g))
    o = plan.forward(qd, kd, vd)
    dq, dk, dv = plan.backward(qd, kd, vd, o, gd)
    torch.cuda.synchronize()
    return [to_np(x) for x in (dq, dk, dv)], plan, (qd, kd, vd, o, gd)


SMALL = [
    # (grid, d, align, tile, custom_b)
    ((3, 5, 20), 128, "frame", 0, 0),    # b=100 (group kernel forward), m=3 (tiny kernel forward)
    ((5, 4, 37), 128, "frame", 0, 0),    # b=148: two key tiles with a ragged tail, m=5
    ((5, 4, 37), 128, "row", 0, 0),      # b=37, m=20
    ((6, 7, 13), 64, "frame", 0, 0),     # d=64
    ((6, 7, 13), 64, "row", 0, 0),
    ((9, 4, 25), 128, "frame", 300, 0),  # tiled: m_tau=3, 3 tiles
    ((10, 15, 8), 128, "row", 0, 0),     # m=150 > 128: stage 2 over several tiles
    ((2, 9, 33), 128, "frame", 0, 0),    # m=2, b=297
    ((3, 5, 20), 128, "dense", 0, 0),    # b=N: one stage
    ((3, 5, 20), 128, "token", 0, 0),    # b=1: stage 2 alone
    ((4, 6, 10), 128, "custom", 0, 20),  # unaligned split
    ((1, 1, 1), 128, "dense", 0, 0),     # one token
    # stage-2 groups of 33..128 rows (one workgroup of ceil(m / 32) waves per group)
    ((81, 2, 3), 128, "frame", 0, 0),    # m=81 (the long layout's group size), three waves
    ((40, 3, 2), 64, "frame", 0, 0),     # m=40, d=64, two waves
    ((128, 1, 3), 128, "frame", 0, 0),   # m=128, four full waves
    ((11, 3, 4), 128, "row", 0, 0),      # m=33: one row in the second wave
    ((96, 2, 2), 128, "frame", 192, 0),  # tiled: m_tau=48 in two tiles
    ((40, 4, 33), 128, "frame", 0, 0),   # b=132 (tiled stage-1 kernels, which read the one-pass
                                         # stage 2's delta), m=40
    ((72, 2, 66), 64, "frame", 0, 0),    # the same with m=72 (three waves), d=64
    # a lone stage of at most 128 rows, done in one pass (final gradients)
    ((2, 4, 12), 128, "dense", 0, 0),    # stage 1 alone, N=96
    ((2, 5, 10), 64, "token", 0, 0),     # stage 2 alone, N=100
]


@pytest.mark.parametrize("grid,d,align,tile,cb", SMALL,
                         ids=[f"{g[0]}x{g[1]}x{g[2]}-d{d}-{a}-t{t}" for g, d, a, t, cb in SMALL])
def test_backward_small_cases(grid, d, align, tile, cb):
    q, k, v = datagen.qkv(2, 3, grid, d, (51, 52, 53), dtype=BF16)
    g = datagen.qkv(2, 3, grid, d, (54, 55, 56), dtype=BF16)[0]
    got, _, _ = grads(q, k, v, g, grid, align, tile, cb)
    b = oracle.block_size(grid, align, cb)
    want = oracle.monarch_backward(q, k, v, g, b, tile or None)
    for name, x, y in zip(("dQ", "dK", "dV"), got, want):
        check(x, y, f"{grid} {align} t{tile} {name}")


@pytest.mark.parametrize("name,heads", [("frame_bf16", 2), ("row_bf16", 2), ("tiled_bf16", 2), ("long_bf16", 1)])
def test_backward_full_size(name, heads):
    c = datagen.CONFIGS[name]
    q, k, v = datagen.config_inputs(name, heads=heads)
    g = datagen.qkv(1, heads, c["grid"], 128, (61, 62, 63), dtype=BF16)[0]
    got, plan, args = grads(q, k, v, g, c["grid"], c["align"], c["tile_tokens"])
    b = oracle.block_size(c["grid"], c["align"])
    want = oracle.monarch_backward(q, k, v, g, b, c["tile_tokens"])
    for nm, x, y in zip(("dQ", "dK", "dV"), got, want):
        check(x, y, f"{name} {nm}")
    # deterministic: no atomics anywhere
    again = plan.backward(*args)
    torch.cuda.synchronize()
    for x, y in zip(got, again):
        assert np.array_equal(x, to_np(y))


@pytest.mark.parametrize("align", ["frame", "row"])
def test_backward_full_grid_head_dim_64(align):
    # the d = 64 backward kernels at full problem length (tiled kernels over 1560-row blocks
    # and 630-row groups, the one-pass kernels for 21-row groups and 52-row blocks), one head
    grid = (21, 30, 52)
    q, k, v = datagen.qkv(1, 1, grid, 64, (4010, 4011, 4012), dtype=BF16)
    g = datagen.qkv(1, 1, grid, 64, (4013, 4014, 4015), dtype=BF16)[0]
    got, _, _ = grads(q, k, v, g, grid, align, 0)
    want = oracle.monarch_backward(q, k, v, g, oracle.block_size(grid, align), None)
    for nm, x, y in zip(("dQ", "dK", "dV"), got, want):
        check(x, y, f"d=64 {align} {nm}")


SAVED = [SMALL[i] for i in (0, 1, 2, 5, 6, 8, 9, 12)] + [((21, 30, 52), 128, "frame", 0, 0)]


@pytest.mark.parametrize("grid,d,align,tile,cb", SAVED,
                         ids=[f"{g[0]}x{g[1]}x{g[2]}-{a}-t{t}" for g, d, a, t, cb in SAVED])
def test_forward_train_and_saved_backward_bitwise(grid, d, align, tile, cb):
    # the training forward runs the backward's recompute launches: its O is
    # bitwise the forward's, and the backward from its saved state is bitwise
    # the recomputing backward (same kernels, same inputs)
    heads = 2 if grid == (21, 30, 52) else 3
    q, k, v = (x.to(DEV) for x in datagen.qkv(1, heads, grid, d, (71, 72, 73), dtype=BF16))
    g = datagen.qkv(1, heads, grid, d, (74, 75, 76), dtype=BF16)[0].to(DEV)
    plan = MonarchPlan(1, heads, d, grid, align=align, tile_tokens=tile, custom_b=cb)
    o = plan.forward(q, k, v)
    o_train, ws = plan.forward_train(q, k, v)
    ref = plan.backward(q, k, v, o, g)
    got = plan.backward(q, k, v, o_train, g, workspace=ws, saved=True)
    torch.cuda.synchronize()
    say(f"  {grid} {align} t{tile}: max |O_train - O| = {(o_train.float() - o.float()).abs().max().item():.1e}")
    assert torch.equal(o_train, o)
    for name, x, y in zip(("dQ", "dK", "dV"), got, ref):
        assert torch.equal(x, y), name
