"""GPU parity of the fused launch (both stages in one persistent kernel).

The fused forward must match the fp64 oracle to the bf16 tolerances, report
no control-block error, be deterministic across calls that reuse one
workspace, and equal the two-launch forward bit for bit where both run the
same stage-2 arithmetic (MFMA groups, 9 <= m_tau <= 32)."""
import numpy as np
import pytest
import torch

import datagen
import oracle
from structured_attention_video_amd import MonarchPlan
from gpu_util import assert_close, guard_intact, guarded_empty, say, to_np

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
BF16 = torch.bfloat16


def fused_and_plain(q, k, v, grid, align="frame", tile=0):
    B, Hh, N, d = q.shape
    fp = MonarchPlan(B, Hh, d, grid, align=align, tile_tokens=tile, dtype=q.dtype, fused=True)
    pp = MonarchPlan(B, Hh, d, grid, align=align, tile_tokens=tile, dtype=q.dtype)
    assert fp.fused, "fused launch expected for this shape"
    say(f"  fused b={fp.info['b']} m_tau={fp.info['m_tau']} tiles={fp.info['tiles']} ws={fp.workspace_bytes}")
    qd, kd, vd = (x.to(DEV) for x in (q, k, v))
    ws = fp.new_workspace(DEV)
    buf, out = guarded_empty(q.shape, q.dtype, DEV)
    fp.forward(qd, kd, vd, out=out, workspace=ws)
    torch.cuda.synchronize()
    assert guard_intact(buf, q.shape), "write past the end of O"
    assert fp.fused_error(ws) == 0, "fused control block reports a wait that timed out"
    plain = pp.forward(qd, kd, vd)
    torch.cuda.synchronize()
    return out.cpu(), plain.cpu(), (fp, qd, kd, vd, ws)


SMALL = [
    # (grid, d, tile) with b = H*W > 128 and 2 <= m_tau <= 32
    ((5, 4, 37), 128, 0),     # b=148, m=5 (unfused stage 2: tiny VALU kernel)
    ((2, 9, 33), 128, 0),     # b=297, m=2
    ((32, 5, 30), 128, 0),    # b=150, m=32 (largest fused group)
    ((12, 5, 30), 128, 0),    # b=150, m=12
    ((6, 6, 25), 128, 300),   # tiled: b=150, m_tau=2, 3 tiles
    ((6, 9, 17), 64, 0),      # d=64, b=153, m=6
    ((10, 9, 17), 64, 0),     # d=64, b=153, m=10
]


@pytest.mark.parametrize("grid,d,tile", SMALL, ids=[f"{g[0]}x{g[1]}x{g[2]}-d{d}-t{t}" for g, d, t in SMALL])
def test_fused_small_cases(grid, d, tile):
    q, k, v = datagen.qkv(2, 3, grid, d, (21, 22, 23), dtype=BF16)
    got, plain, _ = fused_and_plain(q, k, v, grid, "frame", tile)
    b = grid[1] * grid[2]
    assert_close(to_np(got), oracle.monarch_forward(q, k, v, b, tile or None), BF16, f"fused {grid} t{tile}")
    m_tau = (tile or grid[0] * b) // b
    if 9 <= m_tau <= 32:
        assert torch.equal(got, plain), "fused and two-launch forwards differ"
    else:
        assert_close(to_np(got), to_np(plain), BF16, "fused vs two-launch")


@pytest.mark.parametrize("name", ["frame_bf16", "tiled_bf16"])
def test_fused_full_size(name):
    c = datagen.CONFIGS[name]
    q, k, v = datagen.config_inputs(name)
    got, plain, (fp, qd, kd, vd, ws) = fused_and_plain(q, k, v, c["grid"], c["align"], c["tile_tokens"])
    want = oracle.monarch_forward(q, k, v, oracle.block_size(c["grid"], c["align"]), c["tile_tokens"])
    assert_close(to_np(got), want, BF16, f"fused {name}")
    if name == "frame_bf16":
        assert torch.equal(got, plain), "fused and two-launch forwards differ"
    # the same workspace again (control block reset by each call), three times
    outs = [fp.forward(qd, kd, vd, workspace=ws) for _ in range(3)]
    torch.cuda.synchronize()
    assert fp.fused_error(ws) == 0
    assert all(torch.equal(o.cpu(), got) for o in outs)


def test_fused_workspace_reuse_with_new_inputs():
    # Y of the previous call is still in the workspace (and possibly in some
    # XCD's L2): the second call must read its own Y, not the stale one
    grid, d = (12, 5, 30), 128
    a = [x.to(DEV) for x in datagen.qkv(2, 3, grid, d, (31, 32, 33), dtype=BF16)]
    b = [x.to(DEV) for x in datagen.qkv(2, 3, grid, d, (41, 42, 43), dtype=BF16)]
    fp = MonarchPlan(2, 3, d, grid, align="frame", fused=True)
    pp = MonarchPlan(2, 3, d, grid, align="frame")
    ws = fp.new_workspace(DEV)
    for _ in range(3):
        oa = fp.forward(*a, workspace=ws).clone()
        ob = fp.forward(*b, workspace=ws).clone()
        torch.cuda.synchronize()
        assert fp.fused_error(ws) == 0
        assert torch.equal(oa, pp.forward(*a)) and torch.equal(ob, pp.forward(*b))
