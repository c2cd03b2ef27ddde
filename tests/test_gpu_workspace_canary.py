"""NaN-canary workspaces: a call reads only workspace bytes it has written first.

Each case runs the same call twice, once on a workspace filled with 0xFF
bytes (NaN as bf16 and as fp32, -1 as an integer) and once on a zeroed one,
into NaN-prefilled outputs. The results must be finite and bitwise equal: a
kernel that read a workspace element before writing it (Y, the mixed keys and
entropies of the refinement step, a fused plan's control block, the saved
state of the training pair) would carry the canary into its output or differ
between the two runs, and an output row left unwritten stays NaN.
"""
import pytest
import torch

import datagen
from structured_attention_video_amd import MonarchPlan
from gpu_util import say

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
BF16, F32 = torch.bfloat16, torch.float32

FORWARD = [
    # (grid, d, dtype, align, tile, plan kwargs)
    ((5, 4, 37), 128, BF16, "frame", 0, {}),                # flash stage 1, group stage 2
    ((5, 4, 37), 128, BF16, "row", 0, {}),                  # group both stages
    ((10, 15, 8), 128, BF16, "row", 0, {}),                 # group stage 1, flash stage 2 (m = 150)
    ((6, 4, 25), 128, BF16, "frame", 200, {}),              # tiled: tiny stage 2
    ((5, 4, 37), 64, BF16, "frame", 0, {"y_fp32": True}),   # fp32 Y in the workspace
    ((5, 4, 37), 128, BF16, "frame", 0, {"fused": True}),   # control block after Y
    ((5, 4, 37), 128, BF16, "frame", 0, {"refine": True}),  # Y, mixed keys, entropies
    ((10, 15, 8), 128, BF16, "row", 0, {"refine": True}),
    ((5, 4, 37), 128, F32, "frame", 0, {}),                 # generic fp32 kernels
    ((21, 30, 52), 128, BF16, "frame", 0, {}),              # full-size frame grid (two heads)
]


def _canary(n, fill):
    return torch.full((max(n, 1),), fill, dtype=torch.uint8, device=DEV)


def _nan_out(shape, dtype):
    return torch.full(shape, float("nan"), dtype=dtype, device=DEV)


@pytest.mark.parametrize("grid,d,dtype,align,tile,kw", FORWARD,
                         ids=[f"{g[0]}x{g[1]}x{g[2]}-d{d}-{str(t)[6:]}-{a}-t{ti}-{'-'.join(kw) or 'plain'}"
                              for g, d, t, a, ti, kw in FORWARD])
def test_forward_reads_no_unwritten_workspace(grid, d, dtype, align, tile, kw):
    q, k, v = (x.to(DEV) for x in datagen.qkv(1, 2, grid, d, (71, 72, 73), dtype=dtype))
    plan = MonarchPlan(1, 2, d, grid, align=align, tile_tokens=tile, dtype=dtype, **kw)
    n = plan.workspace_bytes
    say(f"  canary forward {grid} {align} t{tile} {kw}: kernels={plan.kernel_names()} ws={n}")
    assert n > 0
    outs = []
    for fill in (0xFF, 0x00):
        o = _nan_out(q.shape, dtype)
        plan.forward(q, k, v, out=o, workspace=_canary(n, fill))
        torch.cuda.synchronize()
        outs.append(o)
    assert torch.isfinite(outs[0]).all(), "canary or unwritten rows reached the output"
    assert torch.equal(outs[0], outs[1]), "the output depends on the workspace's prior contents"
    plan.close()


@pytest.mark.parametrize("grid,align", [((5, 4, 37), "frame"), ((5, 4, 37), "row"), ((10, 15, 8), "row"),
                                        ((4, 6, 30), "frame")])
def test_backward_reads_no_unwritten_workspace(grid, align):
    q, k, v = (x.to(DEV) for x in datagen.qkv(1, 2, grid, 128, (74, 75, 76)))
    g = datagen.qkv(1, 2, grid, 128, (77, 78, 79))[0].to(DEV)
    plan = MonarchPlan(1, 2, 128, grid, align=align)
    o = plan.forward(q, k, v)
    n = plan.backward_workspace_bytes
    say(f"  canary backward {grid} {align}: ws={n}")
    res = []
    for fill in (0xFF, 0x00):
        grads = tuple(_nan_out(q.shape, BF16) for _ in range(3))
        plan.backward(q, k, v, o, g, workspace=_canary(n, fill), grads=grads)
        torch.cuda.synchronize()
        res.append(grads)
    for a, b, name in zip(res[0], res[1], ("dQ", "dK", "dV")):
        assert torch.isfinite(a).all(), f"{name}: canary or unwritten rows"
        assert torch.equal(a, b), f"{name} depends on the workspace's prior contents"
    # the training pair: the forward fills the saved state, the backward reads only that
    saved = []
    for fill in (0xFF, 0x00):
        ws = _canary(n, fill)
        ot, ws = plan.forward_train(q, k, v, out=_nan_out(q.shape, BF16), workspace=ws)
        grads = tuple(_nan_out(q.shape, BF16) for _ in range(3))
        plan.backward(q, k, v, ot, g, workspace=ws, grads=grads, saved=True)
        torch.cuda.synchronize()
        saved.append((ot,) + grads)
    for a, b, name in zip(saved[0], saved[1], ("O", "dQ", "dK", "dV")):
        assert torch.isfinite(a).all(), f"training pair {name}: canary or unwritten rows"
        assert torch.equal(a, b), f"training pair {name} depends on the workspace's prior contents"
    plan.close()
