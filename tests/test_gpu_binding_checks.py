"""The Python binding is the only size guard in front of the C ABI (bare pointers): every
entry point must refuse tensors of the wrong element type or shape before any launch."""
import pytest
import torch

from structured_attention_video_amd import MonarchPlan

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
GRID = (4, 6, 10)


def _t(dtype, n=240):
    return torch.zeros(1, 2, n, 128, dtype=dtype, device=DEV)


def test_forward_and_noalloc_refuse_wrong_types():
    p = MonarchPlan(1, 2, 128, GRID)                                  # bf16 plan
    x, f = _t(torch.bfloat16), _t(torch.float32)
    with pytest.raises(ValueError):
        p.forward(x, x, f)                                            # fp32 v
    with pytest.raises(ValueError):
        p.forward(x, x, x, out=f)                                     # fp32 out: twice the bytes
    with pytest.raises(ValueError):
        p.forward(x, x, x, out=_t(torch.bfloat16, 120))               # short out
    with pytest.raises(ValueError):
        p.forward_noalloc(x, x, x, f)
    with pytest.raises(ValueError):
        p.forward(x, x, x, workspace=torch.empty(10, device="cpu"))   # host workspace


def test_stage_entry_points_refuse_wrong_types():
    p = MonarchPlan(1, 2, 128, GRID)                                  # bf16 plan, bf16 Y
    x, f = _t(torch.bfloat16), _t(torch.float32)
    with pytest.raises(ValueError):
        p.stage1(f, x, x)
    with pytest.raises(ValueError):
        p.stage1(x, x, x, y=f)                                        # Y of the wrong type
    with pytest.raises(ValueError):
        p.stage2(x, x, f)                                             # bf16 plan reads bf16 Y
    with pytest.raises(ValueError):
        p.stage2(x, x, x, out=f)
    with pytest.raises(ValueError):
        p.stage2(x, x, x, out=_t(torch.bfloat16, 120))                # short out
    py = MonarchPlan(1, 2, 128, GRID, y_fp32=True)                    # bf16 plan, fp32 Y
    with pytest.raises(ValueError):
        py.stage2(x, x, x)                                            # a bf16 Y read as fp32: past its end
    py.stage2(x, x, f)                                                # the right type is accepted
    torch.cuda.synchronize()


def test_chunk_and_backward_refuse_wrong_types():
    p = MonarchPlan(1, 2, 128, GRID)
    x, f = _t(torch.bfloat16), _t(torch.float32)
    with pytest.raises(ValueError):
        p.chunk_forward(x, x, x, f, x.clone(), 0, 2)                  # Y of the wrong type
    with pytest.raises(ValueError):
        p.chunk_forward(f, x, x, x.clone(), x.clone(), 0, 2)
    with pytest.raises(ValueError):
        p.backward(x, x, x, x, f)
    with pytest.raises(ValueError):
        p.backward(x, x, x, x, x, grads=(x.clone(), x.clone(), f))


def test_the_in_tree_library_runs_the_forward():
    # the kernels that ran are the in-tree build's: it is mapped into this process, and no
    # other copy of the library is
    import os
    from structured_attention_video_amd import _lib
    p = MonarchPlan(1, 2, 128, GRID)
    x = _t(torch.bfloat16)
    p.forward(x, x, x)
    torch.cuda.synchronize()
    want = os.path.realpath(_lib.LIB_PATH)
    maps = [line.split()[-1] for line in open("/proc/self/maps") if "libmonarch_attn" in line]
    assert maps and all(os.path.realpath(m) == want for m in maps), maps
    assert os.path.dirname(want) == os.path.dirname(os.path.realpath(_lib.__file__))
