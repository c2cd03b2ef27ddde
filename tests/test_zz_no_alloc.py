"""The no-allocation forward (monarch_attn_forward_noalloc) against the ordinary forward.

Both run the same kernels; the no-allocation entry point takes its workspace from the
library's static device array. Two calls in a row, the second on a smaller problem (the
array keeps the first call's contents), then a fused plan; each output must equal the
ordinary forward's bitwise and match the fp64 oracle within the bf16 tolerance."""
import pytest
import torch

import datagen
import oracle
from structured_attention_video_amd import MonarchPlan, MonarchError, _lib
from gpu_util import assert_close, say, to_np

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _both(grid, heads, align="frame", tile=0, fused=False, seeds=(41, 42, 43)):
    q, k, v = datagen.qkv(1, heads, grid, 128, seeds, dtype=torch.bfloat16)
    plan = MonarchPlan(1, heads, 128, grid, align=align, tile_tokens=tile, fused=fused)
    assert 0 < plan.workspace_bytes <= _lib.NOALLOC_SCRATCH_BYTES
    qd, kd, vd = (x.to(DEV) for x in (q, k, v))
    want = plan.forward(qd, kd, vd)
    got = torch.full_like(qd, float("nan"))
    plan.forward_noalloc(qd, kd, vd, got)
    torch.cuda.synchronize()
    say(f"  {grid} heads={heads} {align} tile={tile} fused={plan.fused} ws={plan.workspace_bytes}")
    assert torch.equal(got, want), "no-allocation forward differs from the ordinary forward"
    ref = oracle.monarch_forward(q, k, v, plan.info["b"], tile or None)
    assert_close(to_np(got), ref, torch.bfloat16, f"noalloc {grid} {align}")
    plan.close()


def test_noalloc_matches_forward_two_calls_second_smaller():
    _both((21, 30, 52), 4)            # 4 heads of the frame shape: ~33.5 MB of Y
    _both((5, 6, 20), 2, seeds=(7, 8, 9))  # much smaller: stale contents of the first call remain


def test_noalloc_row_tiled_and_fused():
    _both((6, 10, 52), 2, align="row")
    _both((9, 6, 40), 2, tile=3 * 240)
    _both((7, 8, 40), 3, fused=True)


def test_noalloc_full_frame_shape():
    _both((21, 30, 52), 12)           # the 21x30x52 grid, 12 heads: 100.6 MB of Y


def test_noalloc_rejects_too_large():
    plan = MonarchPlan(1, 12, 128, (81, 30, 52))   # 388 MB of Y
    x = torch.empty(1, 12, 81 * 30 * 52, 128, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(MonarchError) as e:
        plan.forward_noalloc(x, x, x, torch.empty_like(x))
    assert e.value.status == _lib.ERR_TOO_LARGE
    plan.close()
