"""GPU parity: the HIP library through its C ABI against the fp64 oracle.

Small cases span several kernel tiles with ragged tails and are compared on
every element; the named workloads run at full size and are compared in full
(or on sampled stage-2 groups where the oracle would be slow). Tolerances:
bf16 rel-L2 <= 1e-2 and max-abs <= 3e-2, fp32 both <= 1e-5.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import datagen
import oracle
from structured_attention_video_amd import MonarchPlan
from gpu_util import assert_close, errors, guard_intact, guarded_empty, say, to_np

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
BF16, F32 = torch.bfloat16, torch.float32


def run(q, k, v, grid, align="frame", tile=0, custom_b=0, scale=None, **kw):
    """Forward through the C ABI into a guard-banded output; checks the guard."""
    B, Hh, N, d = q.shape
    plan = MonarchPlan(B, Hh, d, grid, align=align, tile_tokens=tile, custom_b=custom_b,
                       dtype=q.dtype, scale=scale, **kw)
    say(f"  plan b={plan.info['b']} m_tau={plan.info['m_tau']} tiles={plan.info['tiles']} "
        f"kernels={plan.kernel_names()}")
    qd, kd, vd = (x.to(DEV) for x in (q, k, v))
    buf, out = guarded_empty(q.shape, q.dtype, DEV)
    plan.forward(qd, kd, vd, out=out)
    torch.cuda.synchronize()
    assert guard_intact(buf, q.shape), "write past the end of O"
    res = out.cpu()
    plan.close()
    return res


def ref(q, k, v, b, tile=0, scale=None):
    return oracle.monarch_forward(q, k, v, b, tile or None, scale)


# ------------------------------------------------------------------ small cases
SMALL = [
    # (grid, d, dtype, align, tile, custom_b)
    ((3, 5, 20), 128, BF16, "frame", 0, 0),     # b=100: ragged against 32/64-row tiles
    ((5, 4, 37), 128, BF16, "frame", 0, 0),     # b=148, m=5
    ((5, 4, 37), 128, BF16, "row", 0, 0),       # b=37, m=20
    ((6, 7, 13), 64, BF16, "frame", 0, 0),      # d=64, b=91
    ((6, 7, 13), 64, BF16, "row", 0, 0),        # d=64, b=13, m=42
    ((6, 4, 25), 128, BF16, "frame", 200, 0),   # tiled: m_tau=2, 3 tiles
    ((9, 4, 25), 128, BF16, "frame", 300, 0),   # tiled: m_tau=3, 3 tiles
    ((10, 15, 8), 128, BF16, "row", 0, 0),      # b=8, m=150 (> 128)
    ((2, 9, 33), 128, BF16, "frame", 0, 0),     # m=2, b=297
    ((2, 10, 27), 128, BF16, "frame", 0, 0),    # b=270: three query tiles of 96 rows, one idle wave each
    ((3, 5, 20), 128, BF16, "dense", 0, 0),     # b=N=300
    ((3, 5, 20), 128, BF16, "token", 0, 0),     # b=1, m=300
    ((4, 6, 10), 128, BF16, "custom", 0, 20),   # unaligned split (ablation)
    ((3, 5, 20), 128, F32, "frame", 0, 0),
    ((5, 4, 37), 64, F32, "row", 0, 0),
    ((6, 4, 25), 128, F32, "frame", 200, 0),
    ((3, 5, 20), 64, F32, "dense", 0, 0),
    ((1, 1, 1), 64, F32, "frame", 0, 0),        # one token: O = V
    ((1, 1, 1), 128, BF16, "dense", 0, 0),
]


@pytest.mark.parametrize("grid,d,dtype,align,tile,cb", SMALL,
                         ids=[f"{g[0]}x{g[1]}x{g[2]}-d{d}-{str(t)[6:]}-{a}-t{ti}" for g, d, t, a, ti, cb in SMALL])
def test_small_cases(grid, d, dtype, align, tile, cb):
    B, Hh = 2, 3
    q, k, v = datagen.qkv(B, Hh, grid, d, (11, 12, 13), dtype=dtype)
    b = oracle.block_size(grid, align, cb)
    got = run(q, k, v, grid, align, tile, cb, allow_unaligned=(align == "custom"))
    assert_close(to_np(got), ref(q, k, v, b, tile), dtype, f"{grid} {align}")


def test_y_fp32_flag():
    grid = (5, 4, 37)
    q, k, v = datagen.qkv(1, 2, grid, 128, (21, 22, 23))
    a = run(q, k, v, grid, "frame")
    b = run(q, k, v, grid, "frame", y_fp32=True)
    want = ref(q, k, v, 148)
    assert_close(to_np(b), want, BF16, "Y fp32")
    # keeping Y in fp32 can only remove rounding
    assert errors(to_np(b), want)[0] <= errors(to_np(a), want)[0] * 1.05


def test_generic_kernel_matches_oracle_bf16():
    grid = (5, 4, 37)
    q, k, v = datagen.qkv(1, 2, grid, 128, (24, 25, 26))
    for align, b in (("frame", 148), ("row", 37)):
        got = run(q, k, v, grid, align, generic=True)
        assert_close(to_np(got), ref(q, k, v, b), BF16, f"generic {align}")


def test_scale_override():
    grid = (4, 6, 10)
    q, k, v = datagen.qkv(1, 2, grid, 64, (27, 28, 29), dtype=F32)
    got = run(q, k, v, grid, "frame", scale=0.05)
    assert_close(to_np(got), ref(q, k, v, 60, 0, 0.05), F32, "scale 0.05")


def test_stage_entry_points_compose():
    grid = (5, 4, 37)
    q, k, v = (x.to(DEV) for x in datagen.qkv(1, 2, grid, 128, (30, 31, 32)))
    plan = MonarchPlan(1, 2, 128, grid)
    y = plan.stage1(q, k, v)
    o2 = plan.stage2(q, k, y)
    o = plan.forward(q, k, v)
    torch.cuda.synchronize()
    assert torch.equal(o, o2)
    # stage 1 alone is block attention: compare Y with the oracle's first factor
    yref = np.stack([oracle.stage1(to_np(q[0, h]), to_np(k[0, h]), to_np(v[0, h]), 148, 128 ** -0.5)
                     for h in range(2)])[None]
    assert_close(to_np(y), yref, BF16, "stage 1")


# ------------------------------------------------------------------ golden (hand-derived)
GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_examples.json")


@pytest.mark.parametrize("ex", json.load(open(GOLDEN))["examples"], ids=lambda e: e["name"])
def test_hand_examples_on_gpu(ex):
    # embed the d=1 examples in d=64: q = e0, k = k_n e0, v = v_n e0, scale 1
    T, H, W = ex["grid"]
    N = T * H * W
    num = lambda s: math.log(int(s[2:])) if s.startswith("ln") else float(Fraction(s))
    q = torch.zeros(1, 1, N, 64)
    k, v = torch.zeros_like(q), torch.zeros_like(q)
    q[..., 0] = 1
    k[0, 0, :, 0] = torch.tensor([num(x) for x in ex["k"]])
    v[0, 0, :, 0] = torch.tensor([num(x) for x in ex["v"]])
    align = "dense" if ex["b"] == N else "frame"
    got = run(q, k, v, ex["grid"], align, ex["tile_tokens"], scale=1.0)
    want = np.array([float(Fraction(x)) for x in ex["o"]])
    np.testing.assert_allclose(to_np(got)[0, 0, :, 0], want, rtol=0, atol=2e-6)
    assert np.all(to_np(got)[0, 0, :, 1:] == 0)


# ------------------------------------------------------------------ the named workloads
def test_tiny_fp32_full_matrix():
    c = datagen.CONFIGS["tiny_fp32"]
    q, k, v = datagen.config_inputs("tiny_fp32")
    got = run(q, k, v, c["grid"], "frame")
    M = oracle.monarch_matrix(q[0, 0], k[0, 0], 64)
    assert_close(to_np(got)[0, 0], M @ to_np(v)[0, 0], F32, "tiny fp32 vs dense N x N matrix")


@pytest.mark.parametrize("name", ["frame_bf16", "row_bf16", "tiled_bf16"])
def test_full_size_workloads(name):
    c = datagen.CONFIGS[name]
    q, k, v = datagen.config_inputs(name)
    got = run(q, k, v, c["grid"], c["align"], c["tile_tokens"])
    b = oracle.block_size(c["grid"], c["align"])
    want = ref(q, k, v, b, c["tile_tokens"])
    assert_close(to_np(got), want, BF16, name)


@pytest.mark.parametrize("align,tile", [("frame", 0), ("row", 0), ("frame", 4680)])
def test_full_grid_head_dim_64(align, tile):
    """The 21x30x52 grid at d = 64, four heads, every element: the d = 64 kernels at full
    problem length (flash over 1560-row blocks and 630-row groups, the short-tile group
    kernel for the 21-row groups, the tiny kernel for tiles of three blocks)."""
    grid = (21, 30, 52)
    q, k, v = datagen.qkv(1, 4, grid, 64, (4000, 4001, 4002))
    got = run(q, k, v, grid, align, tile)
    b = oracle.block_size(grid, align)
    assert_close(to_np(got), ref(q, k, v, b, tile), BF16, f"d=64 {align} t{tile}")


@pytest.mark.parametrize("align", ["frame", "row"])
def test_full_grid_fp32(align):
    """fp32 on the 21x30x52 grid, one head, every element, to the fp32 bound: the generic
    kernel over 1560-key blocks (49 key chunks) and 630-row groups."""
    grid = (21, 30, 52)
    q, k, v = datagen.qkv(1, 1, grid, 128, (4020, 4021, 4022), dtype=F32)
    got = run(q, k, v, grid, align)
    b = oracle.block_size(grid, align)
    assert_close(to_np(got), ref(q, k, v, b), F32, f"fp32 {align}")


def test_long_video_all_heads():
    """The long workload (81 frames, N = 126360) on all 12 heads, every element."""
    c = datagen.CONFIGS["long_bf16"]
    q, k, v = datagen.config_inputs("long_bf16")
    got = run(q, k, v, c["grid"], "frame")
    b = oracle.block_size(c["grid"], "frame")
    for h in range(q.shape[1]):
        want = ref(q[:, h:h + 1], k[:, h:h + 1], v[:, h:h + 1], b)
        assert_close(to_np(got)[:, h:h + 1], want, BF16, f"long video head {h}")


def test_long_dense_kernel_sampled_rows():
    """The dense kernel (b = N) at the long shape on sampled rows, including both ends."""
    c = datagen.CONFIGS["long_bf16"]
    q, k, v = datagen.config_inputs("long_bf16", heads=1)
    got = run(q, k, v, c["grid"], "dense")
    N = q.shape[2]
    rows = np.concatenate([[0, 1, N - 2, N - 1], np.random.default_rng(8).integers(0, N, 60)])
    want = oracle.dense_attention(q[0, 0], k[0, 0], v[0, 0], rows=rows)
    assert_close(to_np(got)[0, 0, rows], want, BF16, "long dense head 0")


def test_dense_kernel_sampled_rows():
    c = datagen.CONFIGS["frame_bf16"]
    q, k, v = datagen.config_inputs("frame_bf16", heads=2)
    got = run(q, k, v, c["grid"], "dense")
    rows = np.concatenate([[0, 1, 32759], np.random.default_rng(6).integers(0, 32760, 125)])
    for h in range(2):
        want = oracle.dense_attention(q[0, h], k[0, h], v[0, h], rows=rows)
        assert_close(to_np(got)[0, h, rows], want, BF16, f"dense head {h}")


@pytest.mark.parametrize("align,tile", [("frame", 0), ("row", 0), ("frame", 4680)])
def test_separable_full_size_matches_dense(align, tile):
    grid = (21, 30, 52)
    q, k, v = datagen.separable_qkv(1, 2, grid, 128, 3000)
    got = run(q, k, v, grid, align, tile)
    # aligned Monarch is exact for separable logits: compare with dense (or tile-masked dense)
    rows = np.random.default_rng(7).integers(0, 32760, 96)
    for h in range(2):
        want = oracle.dense_attention(q[0, h], k[0, h], v[0, h], rows=rows, key_tile=tile or None)
        assert_close(to_np(got)[0, h, rows], want, BF16, f"separable {align} t{tile} head {h}")
    if not tile:
        dense = run(q, k, v, grid, "dense")
        assert_close(to_np(got), to_np(dense), BF16, "separable Monarch vs GPU dense kernel")


def test_zero_queries_give_tile_mean_full_size():
    c = datagen.CONFIGS["tiled_bf16"]
    q, k, v = datagen.config_inputs("tiled_bf16", heads=2)
    q = torch.zeros_like(q)
    got = run(q, k, v, c["grid"], "frame", 4680)
    vv = to_np(v)[0]
    want = np.repeat(vv.reshape(2, 7, 4680, 128).mean(axis=2), 4680, axis=1)
    assert_close(to_np(got)[0], want, BF16, "Q=0 tile mean")


def test_inblock_permutation_equivariance_full_size():
    c = datagen.CONFIGS["frame_bf16"]
    q, k, v = datagen.config_inputs("frame_bf16", heads=2)
    b = 1560
    sigma = torch.from_numpy(np.random.default_rng(8).permutation(b))
    n = torch.arange(32760)
    perm = (n // b) * b + sigma[n % b]
    o = run(q, k, v, c["grid"], "frame")
    op = run(q[:, :, perm], k[:, :, perm], v[:, :, perm], c["grid"], "frame")
    assert_close(to_np(op), to_np(o[:, :, perm]), BF16, "permuted blocks")


def test_stage1_full_size_all_heads():
    # the first factor alone, every head of the frame workload (stage 2 would
    # average errors over 21 blocks and hide a wrong row)
    q, k, v = datagen.config_inputs("frame_bf16")
    plan = MonarchPlan(1, 12, 128, (21, 30, 52), align="frame")
    y = plan.stage1(q.to(DEV), k.to(DEV), v.to(DEV))
    torch.cuda.synchronize()
    Y = to_np(y)[0]
    for h in range(12):
        yref = oracle.stage1(to_np(q[0, h]), to_np(k[0, h]), to_np(v[0, h]), 1560, 128 ** -0.5)
        assert_close(Y[h], yref, BF16, f"stage 1 head {h}")


@pytest.mark.parametrize("name", ["frame_bf16", "tiled_bf16", "row_bf16"])
def test_forward_is_deterministic(name):
    c = datagen.CONFIGS[name]
    q, k, v = (x.to(DEV) for x in datagen.config_inputs(name))
    plan = MonarchPlan(1, 12, 128, c["grid"], align=c["align"], tile_tokens=c["tile_tokens"])
    outs = [plan.forward(q, k, v) for _ in range(3)]
    y = plan.stage1(q, k, v)
    o2 = plan.stage2(q, k, y)
    torch.cuda.synchronize()
    assert all(torch.equal(outs[0], o) for o in outs[1:])
    assert torch.equal(outs[0], o2)
