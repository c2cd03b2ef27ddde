"""GPU parity of the one-refinement-step forward (MONARCH_FLAG_REFINE) against the
fp64 refinement oracle (oracle/monarch_refine.py, one step from an identity stage-2
factor). Same tolerances as the direct forward: bf16 rel-L2 <= 1e-2 and max-abs <=
3e-2, fp32 both <= 1e-5. Small cases span several kernel tiles with ragged tails;
the 21x30x52 workloads run at full size."""
import numpy as np
import pytest
import torch

import datagen
import oracle
from structured_attention_video_amd import MonarchPlan
from gpu_util import assert_close, guard_intact, guarded_empty, say, to_np

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
BF16, F32 = torch.bfloat16, torch.float32


def run(q, k, v, grid, align="frame", tile=0, custom_b=0, **kw):
    B, Hh, N, d = q.shape
    plan = MonarchPlan(B, Hh, d, grid, align=align, tile_tokens=tile, custom_b=custom_b, dtype=q.dtype,
                       refine=True, **kw)
    say(f"  plan b={plan.info['b']} m_tau={plan.info['m_tau']} refine={plan.info['refine_steps']} "
        f"kernels={plan.kernel_names()} ws={plan.workspace_bytes}")
    qd, kd, vd = (x.to(DEV) for x in (q, k, v))
    buf, out = guarded_empty(q.shape, q.dtype, DEV)
    plan.forward(qd, kd, vd, out=out)
    torch.cuda.synchronize()
    assert guard_intact(buf, q.shape), "write past the end of O"
    res = out.cpu()
    plan.close()
    return res


SMALL = [
    # (grid, d, dtype, align, tile, custom_b)
    ((3, 5, 20), 128, BF16, "frame", 0, 0),     # b=100 (group kernel stage 1), m=3 (tiny stage 2)
    ((5, 4, 37), 128, BF16, "frame", 0, 0),     # b=148 (flash stage 1 with entropies), m=5
    ((12, 5, 30), 128, BF16, "frame", 0, 0),    # b=150, m=12 (group kernel stage 2 with key biases)
    ((40, 3, 50), 128, BF16, "frame", 0, 0),    # b=150, m=40: two 32-row waves in stage 2
    ((5, 4, 37), 128, BF16, "row", 0, 0),       # b=37, m=20
    ((10, 15, 8), 128, BF16, "row", 0, 0),      # b=8, m=150 > 128 (flash stage 2 with key biases, 22-key last tile)
    ((20, 10, 6), 128, BF16, "row", 0, 0),      # b=6, m=200: four key tiles, 8 keys in the last
    ((9, 20, 6), 64, BF16, "row", 0, 0),        # d=64, b=6, m=180 (flash stage 2, d=64)
    ((6, 7, 13), 64, BF16, "frame", 0, 0),      # d=64, b=91
    ((6, 7, 40), 64, BF16, "frame", 0, 0),      # d=64, b=280 (flash, d=64)
    ((6, 4, 25), 128, BF16, "frame", 200, 0),   # tiled: m_tau=2, 3 tiles
    ((9, 6, 30), 128, BF16, "frame", 540, 0),   # tiled: b=180, m_tau=3
    ((4, 6, 10), 128, BF16, "custom", 0, 20),   # unaligned split (ablation)
    ((3, 5, 20), 128, F32, "frame", 0, 0),
    ((5, 4, 37), 64, F32, "row", 0, 0),
    ((6, 4, 25), 128, F32, "frame", 200, 0),
]


@pytest.mark.parametrize("grid,d,dtype,align,tile,cb", SMALL,
                         ids=[f"{g[0]}x{g[1]}x{g[2]}-d{d}-{str(t)[6:]}-{a}-t{ti}" for g, d, t, a, ti, cb in SMALL])
def test_refine_small_cases(grid, d, dtype, align, tile, cb):
    q, k, v = datagen.qkv(2, 3, grid, d, (51, 52, 53), dtype=dtype)
    b = oracle.block_size(grid, align, cb)
    got = run(q, k, v, grid, align, tile, cb, allow_unaligned=(align == "custom"))
    want = oracle.monarch_refine_forward(q, k, v, b, tile or None)
    assert_close(to_np(got), want, dtype, f"refine {grid} {align} t{tile}")
    # the step changes the result: it is not the direct forward
    direct = oracle.monarch_forward(q, k, v, b, tile or None)
    assert np.abs(want - direct).max() > 1e-3


@pytest.mark.parametrize("grid,align", [((5, 4, 37), "frame"), ((10, 15, 8), "row")])
def test_refine_generic_kernels(grid, align):
    q, k, v = datagen.qkv(1, 2, grid, 128, (54, 55, 56), dtype=BF16)
    got = run(q, k, v, grid, align, generic=True)
    b = oracle.block_size(grid, align)
    assert_close(to_np(got), oracle.monarch_refine_forward(q, k, v, b), BF16, f"refine generic {align}")


@pytest.mark.parametrize("align", ["dense", "token"])
def test_refine_degenerate_equals_direct(align):
    grid = (3, 5, 20)
    q, k, v = datagen.qkv(1, 2, grid, 128, (57, 58, 59), dtype=BF16)
    B, Hh, N, d = q.shape
    p = MonarchPlan(B, Hh, d, grid, align=align, refine=True)
    assert p.info["refine_steps"] == 0
    qd, kd, vd = (x.to(DEV) for x in (q, k, v))
    a = p.forward(qd, kd, vd)
    b = MonarchPlan(B, Hh, d, grid, align=align).forward(qd, kd, vd)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


@pytest.mark.parametrize("name", ["frame_bf16", "row_bf16", "tiled_bf16"])
def test_refine_full_size(name):
    c = datagen.CONFIGS[name]
    q, k, v = datagen.config_inputs(name)
    got = run(q, k, v, c["grid"], c["align"], c["tile_tokens"] or 0)
    b = oracle.block_size(c["grid"], c["align"])
    heads = [0, 5, 11]
    want = oracle.monarch_refine_forward(q[0, heads], k[0, heads], v[0, heads], b, c["tile_tokens"])
    assert_close(to_np(got[0, heads]), want, BF16, f"refine {name} heads {heads}")


def test_refine_long_one_head():
    # the long workload (81 frames, m = 81: stage 2 in the group kernel with key biases), head 0
    c = datagen.CONFIGS["long_bf16"]
    q, k, v = datagen.config_inputs("long_bf16", heads=1)
    got = run(q, k, v, c["grid"], "frame")
    want = oracle.monarch_refine_forward(q[0], k[0], v[0], oracle.block_size(c["grid"], "frame"), None)
    assert_close(to_np(got[0]), want, BF16, "refine long head 0")


def test_refine_separable_full_size_matches_dense():
    """Aligned blocks keep separable logits exactly (explainer section 2.A), so the refined
    factors give dense attention at the 21x30x52 grid; compared with the library's dense kernel
    and with the fp64 dense oracle on sampled rows."""
    grid = (21, 30, 52)
    q, k, v = datagen.separable_qkv(1, 2, grid, 128, 3000)
    got = run(q, k, v, grid, "frame")
    qd, kd, vd = (x.to(DEV) for x in (q, k, v))
    dense = MonarchPlan(1, 2, 128, grid, align="dense").forward(qd, kd, vd).cpu()
    assert_close(to_np(got), to_np(dense), BF16, "refine vs dense kernel")
    rows = np.random.default_rng(0).choice(q.shape[2], 256, replace=False)
    want = oracle.dense_attention(q[0, 0], k[0, 0], v[0, 0], rows=rows)
    assert_close(to_np(got[0, 0, rows]), want, BF16, "refine vs dense oracle (sampled rows)")
