"""C-ABI checks that need no GPU: exported symbols, plan arithmetic, and every
validation error path. Pointer arguments here are fake addresses that the
library must reject before any HIP call; no case reaches a launch."""
import ctypes
import os
import re

import pytest

import oracle
from structured_attention_video_amd import _lib, MonarchPlan, MonarchError

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
L = _lib.lib()


def _declared_functions():
    names = set()
    for f in os.listdir(os.path.join(ROOT, "include")):
        if f.endswith(".h"):
            src = open(os.path.join(ROOT, "include", f)).read()
            src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
            names |= set(re.findall(r"\b(monarch_\w+)\s*\(", src))
    return names


def test_every_declared_symbol_is_exported():
    declared = _declared_functions()
    assert declared == set(_lib.EXPORTED)
    for name in declared:
        assert hasattr(L, name), name
    assert L.monarch_attn_abi_version() == 5


def _plan(batch=1, heads=2, d=128, grid=(4, 6, 10), align=0, custom_b=0, tile=0, dtype=0,
          scale=0.0, flags=0):
    h = ctypes.c_void_p(123)
    st = L.monarch_attn_plan(ctypes.byref(h), batch, heads, d, *grid, align, custom_b, tile, dtype,
                             scale, flags)
    return st, h


@pytest.mark.parametrize("kw,status", [
    (dict(batch=0), _lib.ERR_INVALID_ARG),
    (dict(heads=-1), _lib.ERR_INVALID_ARG),
    (dict(grid=(0, 6, 10)), _lib.ERR_INVALID_ARG),
    (dict(dtype=7), _lib.ERR_INVALID_ARG),
    (dict(align=9), _lib.ERR_INVALID_ARG),
    (dict(flags=1 << 20), _lib.ERR_INVALID_ARG),
    (dict(scale=float("nan")), _lib.ERR_INVALID_ARG),
    (dict(scale=-0.5), _lib.ERR_INVALID_ARG),
    (dict(tile=-5), _lib.ERR_INVALID_ARG),
    (dict(grid=(2048, 1024, 1024)), _lib.ERR_INVALID_ARG),  # N >= 2^31
    (dict(d=96), _lib.ERR_UNSUPPORTED),
    (dict(d=256), _lib.ERR_UNSUPPORTED),
    (dict(align=4, custom_b=0), _lib.ERR_INVALID_ARG),
    (dict(align=4, custom_b=7), _lib.ERR_UNALIGNED),       # 7 does not divide 240
    (dict(align=4, custom_b=20), _lib.ERR_UNALIGNED),      # 2W cuts the h axis
    (dict(tile=100), _lib.ERR_UNALIGNED),                  # not whole frames
    (dict(tile=180), _lib.ERR_UNALIGNED),                  # 3 frames do not divide 4
])
def test_plan_errors(kw, status):
    st, h = _plan(**kw)
    assert st == status
    assert h.value is None


def test_plan_null_out():
    assert L.monarch_attn_plan(None, 1, 1, 64, 2, 2, 2, 0, 0, 0, 0, 0.0, 0) == _lib.ERR_INVALID_ARG


@pytest.mark.parametrize("name,b,m_tau,tiles", [
    ("tiny_fp32", 64, 8, 1),
    ("frame_bf16", 1560, 21, 1),
    ("row_bf16", 52, 630, 1),
    ("tiled_bf16", 1560, 3, 7),
    ("long_bf16", 1560, 81, 1),
])
def test_plan_info_for_the_workloads(name, b, m_tau, tiles):
    import datagen
    c = datagen.CONFIGS[name]
    p = MonarchPlan(c["batch"], c["heads"], c["d"], c["grid"], align=c["align"],
                    tile_tokens=c["tile_tokens"], dtype=c["dtype"])
    i = p.info
    assert (i["b"], i["m_tau"], i["tiles"]) == (b, m_tau, tiles)
    N = i["N"]
    assert oracle.block_size(c["grid"], c["align"]) == b
    want = oracle.flop_count(c["batch"], c["heads"], N, c["d"], b, m_tau)
    assert i["flops_stage1"] + i["flops_stage2"] == want
    esz = 4 if c["dtype"] == "fp32" else 2
    assert p.workspace_bytes == c["batch"] * c["heads"] * N * c["d"] * esz
    assert abs(i["scale"] - c["d"] ** -0.5) < 1e-7
    p.close()


def test_identity_factors_need_no_workspace():
    for align, tile in [("dense", 0), ("token", 0), ("frame", 60)]:
        p = MonarchPlan(1, 1, 64, (4, 6, 10), align=align, tile_tokens=tile, dtype="fp32")
        assert p.workspace_bytes == 0
        s1, s2 = p.kernel_names()
        if align == "token":
            assert s1 == "none" and s2 != "none"
        else:
            assert s2 == "none" and s1 != "none"
        p.close()


def test_custom_unaligned_needs_flag():
    with pytest.raises(MonarchError):
        MonarchPlan(1, 1, 64, (4, 6, 10), align="custom", custom_b=20)
    p = MonarchPlan(1, 1, 64, (4, 6, 10), align="custom", custom_b=20, allow_unaligned=True)
    assert p.info["b"] == 20 and p.info["m_tau"] == 12
    # aligned custom sizes need no flag
    for b in (1, 10, 60, 240):
        MonarchPlan(1, 1, 64, (4, 6, 10), align="custom", custom_b=b).close()


def test_y_fp32_flag():
    p = MonarchPlan(1, 1, 128, (4, 6, 10), y_fp32=True)
    assert p.info["y_dtype"] == _lib.FP32 and p.workspace_bytes == 240 * 128 * 4


# ------------------------------------------------------------- forward error paths
A = 0x7f0000000000          # fake, never dereferenced
STEP = 1 << 24              # far apart: no accidental overlap


@pytest.fixture
def plan():
    st, h = _plan(heads=2, grid=(4, 6, 10))  # bf16, N = 240, d = 128
    assert st == _lib.OK
    yield h
    L.monarch_attn_destroy(h)


def _fwd(h, q=A, k=A + STEP, v=A + 2 * STEP, o=A + 3 * STEP, ws=A + 4 * STEP, ws_n=1 << 30):
    return L.monarch_attn_forward(h, q, k, v, o, ws, ws_n, None)


def test_forward_errors(plan):
    io = 2 * 240 * 128 * 2
    assert _fwd(None) == _lib.ERR_INVALID_ARG
    assert _fwd(plan, q=None) == _lib.ERR_INVALID_ARG
    assert _fwd(plan, o=None) == _lib.ERR_INVALID_ARG
    assert _fwd(plan, k=A + STEP + 2) == _lib.ERR_UNALIGNED
    assert _fwd(plan, ws=None) == _lib.ERR_WORKSPACE
    assert _fwd(plan, ws_n=io - 1) == _lib.ERR_WORKSPACE
    assert _fwd(plan, ws=A + 4 * STEP + 8) == _lib.ERR_UNALIGNED
    assert _fwd(plan, o=A + 16) == _lib.ERR_ALIAS                    # o overlaps q
    assert _fwd(plan, o=A + 2 * STEP + io - 16) == _lib.ERR_ALIAS    # o tail overlaps v
    assert _fwd(plan, ws=A + 3 * STEP + 64) == _lib.ERR_ALIAS        # workspace overlaps o
    assert _fwd(plan, ws=A + STEP) == _lib.ERR_ALIAS                 # workspace overlaps k


def test_noalloc_forward_errors(plan):
    """Argument errors of the no-allocation forward return before any HIP call."""
    fwd = L.monarch_attn_forward_noalloc
    assert fwd(None, A, A + STEP, A + 2 * STEP, A + 3 * STEP, None) == _lib.ERR_INVALID_ARG
    assert fwd(plan, A, A + STEP, A + 2 * STEP, None, None) == _lib.ERR_INVALID_ARG
    assert fwd(plan, A, A + STEP + 8, A + 2 * STEP, A + 3 * STEP, None) == _lib.ERR_UNALIGNED
    assert fwd(plan, A, A + STEP, A + 2 * STEP, A + 16, None) == _lib.ERR_ALIAS
    # 12 heads of the 81x30x52 grid: 388 MB of Y, more than the static scratch
    st, big = _plan(heads=12, grid=(81, 30, 52))
    assert st == _lib.OK and L.monarch_attn_workspace_size(big) > _lib.NOALLOC_SCRATCH_BYTES
    assert fwd(big, A, A + (1 << 32), A + (2 << 32), A + (3 << 32), None) == _lib.ERR_TOO_LARGE
    L.monarch_attn_destroy(big)
    # 12 heads of the 21x30x52 grid fit (100.6 MB)
    st, frame = _plan(heads=12, grid=(21, 30, 52))
    assert L.monarch_attn_workspace_size(frame) <= _lib.NOALLOC_SCRATCH_BYTES
    L.monarch_attn_destroy(frame)


def test_stage_entry_errors(plan):
    io = 2 * 240 * 128 * 2
    assert L.monarch_attn_stage1(plan, A, A + STEP, A + 2 * STEP, None, io, None) == _lib.ERR_INVALID_ARG
    assert L.monarch_attn_stage1(plan, A, A + STEP, A + 2 * STEP, A + 3 * STEP, io - 2, None) == _lib.ERR_WORKSPACE
    assert L.monarch_attn_stage1(plan, A, A + STEP, A + 2 * STEP, A + 2 * STEP, io, None) == _lib.ERR_ALIAS
    assert L.monarch_attn_stage2(plan, A, A + STEP, A + 2 * STEP, A + 2 * STEP + 32, None) == _lib.ERR_ALIAS
    assert L.monarch_attn_stage2(plan, A, A + STEP, A + 2 * STEP + 4, A + 3 * STEP, None) == _lib.ERR_UNALIGNED
    st, dense = _plan(grid=(4, 6, 10), align=2)
    assert L.monarch_attn_stage2(dense, A, A + STEP, A + 2 * STEP, A + 3 * STEP, None) == _lib.ERR_INVALID_ARG
    L.monarch_attn_destroy(dense)
    st, tok = _plan(grid=(4, 6, 10), align=3)
    assert L.monarch_attn_stage1(tok, A, A + STEP, A + 2 * STEP, A + 3 * STEP, io, None) == _lib.ERR_INVALID_ARG
    L.monarch_attn_destroy(tok)


def test_status_strings_and_kernel_names():
    for code in range(8):
        assert L.monarch_status_string(code)
    assert L.monarch_status_string(99) == b"unknown status"
    for kid in range(6):
        assert L.monarch_attn_kernel_name(kid)
    assert L.monarch_attn_plan_info(None, None) == _lib.ERR_INVALID_ARG
    assert L.monarch_attn_workspace_size(None) == 0
    L.monarch_attn_destroy(None)


def test_binding_refuses_cpu_tensors():
    import torch
    p = MonarchPlan(1, 1, 64, (2, 2, 2), dtype="fp32")
    x = torch.zeros(1, 1, 8, 64)
    with pytest.raises(ValueError):
        p.forward(x, x, x)


# ------------------------------------------------------------------ fused plans
def _info(**kw):
    st, h = _plan(**kw)
    assert st == _lib.OK
    info = _lib.PlanInfo()
    assert L.monarch_attn_plan_info(h, ctypes.byref(info)) == _lib.OK
    ws = L.monarch_attn_workspace_size(h)
    L.monarch_attn_destroy(h)
    return info, ws


def test_fused_plan_applies_to_frame_and_tiled_bf16():
    # frame 21x30x52: b = 1560 > 128 (flash stage 1), m = 21 <= 32 (one-wave groups)
    info, ws = _info(heads=12, grid=(21, 30, 52), flags=_lib.FLAG_FUSED)
    assert info.fused == 1
    y = 12 * 32760 * 128 * 2
    assert ws == (y + 255) // 256 * 256 + (32 + 32 * 12 * 1) * 4
    # the separate stages keep their own kernels (stage1/stage2 entry points)
    assert L.monarch_attn_kernel_name(info.stage1_kernel) == b"flash_mfma_bf16"
    info, ws = _info(heads=12, grid=(21, 30, 52), tile=4680, flags=_lib.FLAG_FUSED)
    assert info.fused == 1 and info.tiles == 7
    assert ws == (y + 255) // 256 * 256 + (32 + 32 * 12 * 7) * 4
    assert L.monarch_attn_kernel_name(5) == b"fused_mfma_bf16"


@pytest.mark.parametrize("kw", [
    dict(heads=12, grid=(21, 30, 52), align=1),                          # row: b = 52 (group stage 1)
    dict(heads=12, grid=(81, 30, 52)),                                   # m = 81 > 32
    dict(heads=2, grid=(21, 30, 52), dtype=1),                           # fp32
    dict(heads=2, grid=(21, 30, 52), flags=_lib.FLAG_Y_FP32),            # Y fp32
    dict(heads=2, grid=(21, 30, 52), flags=_lib.FLAG_GENERIC),           # diagnostics path
    dict(heads=2, grid=(21, 30, 52), align=2),                           # dense: no stage 2
], ids=["row", "m81", "fp32", "y_fp32", "generic", "dense"])
def test_fused_flag_ignored_where_it_does_not_apply(kw):
    flags = kw.pop("flags", 0) | _lib.FLAG_FUSED
    info, ws = _info(flags=flags, **kw)
    assert info.fused == 0
    plain, ws_plain = _info(flags=flags & ~_lib.FLAG_FUSED, **kw)
    assert ws == ws_plain


# ------------------------------------------------------------------ backward
def test_backward_workspace_size():
    st, h = _plan(heads=12, grid=(21, 30, 52))
    n = L.monarch_attn_backward_workspace_size(h)
    rows = 12 * 32760 * 4
    t2, t4 = 12 * 32760 * 128 * 2, 12 * 32760 * 128 * 4
    up = lambda x: (x + 255) // 256 * 256
    assert n == 2 * up(t2) + 2 * up(t4) + 4 * up(rows)
    L.monarch_attn_destroy(h)
    for kw in (dict(dtype=1), dict(flags=_lib.FLAG_GENERIC)):
        st, h = _plan(**kw)
        assert st == _lib.OK and L.monarch_attn_backward_workspace_size(h) == 0
        L.monarch_attn_destroy(h)


def test_backward_argument_errors():
    F = 1 << 36  # fake, 16-byte aligned device addresses, never dereferenced
    st, h = _plan(heads=2, grid=(4, 6, 10))
    n = L.monarch_attn_backward_workspace_size(h)
    io = 2 * 240 * 128 * 2
    ptr = [F + i * (1 << 30) for i in range(9)]
    ws = F + 20 * (1 << 30)
    call = lambda p, wsz=n, w=ws: L.monarch_attn_backward(h, *p, w, wsz, None)
    assert call([0] + ptr[1:8]) == _lib.ERR_INVALID_ARG
    assert call(ptr[:8], w=0) == _lib.ERR_INVALID_ARG
    assert call(ptr[:8], wsz=n - 1) == _lib.ERR_WORKSPACE
    assert call([ptr[0] + 4] + ptr[1:8]) == _lib.ERR_UNALIGNED
    assert call(ptr[:5] + [ptr[0] + 64] + ptr[6:8]) == _lib.ERR_ALIAS        # grad_q overlaps q
    assert call(ptr[:6] + [ptr[5] + io - 16, ptr[7]]) == _lib.ERR_ALIAS       # grad_k overlaps grad_q
    assert call(ptr[:8], w=ptr[7] + 32) == _lib.ERR_ALIAS                      # workspace overlaps grad_v
    L.monarch_attn_destroy(h)
    st, h = _plan(heads=2, grid=(4, 6, 10), dtype=1)
    assert L.monarch_attn_backward(h, *ptr[:8], ws, 1 << 30, None) == _lib.ERR_UNSUPPORTED
    L.monarch_attn_destroy(h)


def test_backward_saved_argument_errors():
    F = 1 << 36
    st, h = _plan(heads=2, grid=(4, 6, 10))
    n = L.monarch_attn_backward_workspace_size(h)
    io = 2 * 240 * 128 * 2
    ptr = [F + i * (1 << 30) for i in range(9)]
    ws = F + 20 * (1 << 30)
    call = lambda p, wsz=n, w=ws: L.monarch_attn_backward_saved(h, *p, w, wsz, None)
    assert call([0] + ptr[1:8]) == _lib.ERR_INVALID_ARG
    assert call(ptr[:8], w=0) == _lib.ERR_INVALID_ARG
    assert call(ptr[:8], wsz=n - 1) == _lib.ERR_WORKSPACE
    assert call([ptr[0] + 4] + ptr[1:8]) == _lib.ERR_UNALIGNED
    assert call(ptr[:5] + [ptr[0] + 64] + ptr[6:8]) == _lib.ERR_ALIAS        # grad_q overlaps q
    assert call(ptr[:8], w=ptr[7] + 32) == _lib.ERR_ALIAS                      # workspace overlaps grad_v
    L.monarch_attn_destroy(h)
    st, h = _plan(heads=2, grid=(4, 6, 10), dtype=1)
    assert L.monarch_attn_backward_saved(h, *ptr[:8], ws, 1 << 30, None) == _lib.ERR_UNSUPPORTED
    L.monarch_attn_destroy(h)


def test_forward_train_argument_errors():
    F = 1 << 36
    st, h = _plan(heads=2, grid=(4, 6, 10))
    n = L.monarch_attn_backward_workspace_size(h)
    io = 2 * 240 * 128 * 2
    q, k, v, o = (F + i * (1 << 30) for i in range(4))
    ws = F + 20 * (1 << 30)
    call = lambda *a, w=ws, wsz=n: L.monarch_attn_forward_train(h, *a, w, wsz, None)
    assert call(0, k, v, o) == _lib.ERR_INVALID_ARG
    assert call(q, k, v, 0) == _lib.ERR_INVALID_ARG
    assert call(q, k, v, o, w=0) == _lib.ERR_INVALID_ARG
    assert call(q, k, v, o, wsz=n - 1) == _lib.ERR_WORKSPACE
    assert call(q, k + 8, v, o) == _lib.ERR_UNALIGNED
    assert call(q, k, v, o, w=ws + 8) == _lib.ERR_UNALIGNED
    assert call(q, k, v, v + io - 16) == _lib.ERR_ALIAS                      # o overlaps v
    assert call(q, k, v, o, w=q + 256) == _lib.ERR_ALIAS                    # workspace overlaps q
    assert call(q, k, v, ws + n - 16) == _lib.ERR_ALIAS                     # o overlaps the workspace
    L.monarch_attn_destroy(h)
    for kw in (dict(dtype=1), dict(flags=_lib.FLAG_GENERIC)):
        st, h = _plan(heads=2, grid=(4, 6, 10), **kw)
        assert L.monarch_attn_forward_train(h, q, k, v, o, ws, 1 << 30, None) == _lib.ERR_UNSUPPORTED
        L.monarch_attn_destroy(h)


# ------------------------------------------------------------------ chunk forward
def test_chunk_forward_argument_errors():
    F = 1 << 36
    ptr = [F + i * (1 << 30) for i in range(5)]  # q, k, v, y, o
    st, h = _plan(heads=2, grid=(4, 6, 10))
    call = lambda t0, t1, p=ptr: L.monarch_attn_chunk_forward(h, t0, t1, *p, None)
    assert call(-1, 2) == _lib.ERR_INVALID_ARG
    assert call(2, 2) == _lib.ERR_INVALID_ARG
    assert call(1, 5) == _lib.ERR_INVALID_ARG          # t1 > T
    assert call(0, 2, [0] + ptr[1:]) == _lib.ERR_INVALID_ARG
    assert call(0, 2, ptr[:3] + [0, ptr[4]]) == _lib.ERR_INVALID_ARG   # y needed when b > 1
    assert call(0, 2, [ptr[0] + 2] + ptr[1:]) == _lib.ERR_UNALIGNED
    assert call(0, 2, ptr[:4] + [ptr[1] + 64]) == _lib.ERR_ALIAS       # o overlaps k
    L.monarch_attn_destroy(h)
    for kw in (dict(tile=120), dict(align=2)):  # tiled; dense (one block = the whole video)
        st, h = _plan(heads=2, grid=(4, 6, 10), **kw)
        assert st == _lib.OK
        assert L.monarch_attn_chunk_forward(h, 0, 2, *ptr, None) == _lib.ERR_UNSUPPORTED
        L.monarch_attn_destroy(h)


# ------------------------------------------------------------------ refinement step
def test_refine_plan_info_and_workspace():
    a256 = lambda x: (x + 255) // 256 * 256
    info, ws = _info(heads=12, grid=(21, 30, 52), flags=_lib.FLAG_REFINE)
    assert info.refine_steps == 1 and info.fused == 0 and info.fused_error_offset == -1
    t = 12 * 32760 * 128 * 2
    assert ws == a256(t) + a256(t) + a256(12 * 32760 * 4)      # Y, mixed keys, entropies
    info, ws = _info(heads=2, grid=(4, 6, 10), flags=_lib.FLAG_REFINE | _lib.FLAG_Y_FP32)
    assert ws == a256(2 * 240 * 128 * 4) + a256(2 * 240 * 128 * 2) + a256(2 * 240 * 4)
    # the fused flag is overridden
    info, _ = _info(heads=2, grid=(4, 6, 10), flags=_lib.FLAG_REFINE | _lib.FLAG_FUSED)
    assert info.refine_steps == 1 and info.fused == 0
    # nothing to refine with one factor the identity
    for align in (2, 3):
        info, ws = _info(heads=2, grid=(4, 6, 10), align=align, flags=_lib.FLAG_REFINE)
        assert info.refine_steps == 0 and ws == 0


def test_refine_stage2_kernel_supports_key_biases():
    # m_tau = 3 (tiny), 12 (group) and 150 (> 128: flash) with key biases; fp32 and the
    # generic flag take the generic kernel
    info, _ = _info(heads=1, grid=(3, 5, 20), flags=_lib.FLAG_REFINE)
    assert L.monarch_attn_kernel_name(info.stage2_kernel) == b"tiny_group_valu"
    info, _ = _info(heads=1, grid=(12, 5, 30), flags=_lib.FLAG_REFINE)
    assert L.monarch_attn_kernel_name(info.stage2_kernel) == b"small_group_mfma_bf16"
    info, _ = _info(heads=1, grid=(10, 15, 8), align=1, flags=_lib.FLAG_REFINE)
    assert L.monarch_attn_kernel_name(info.stage2_kernel) == b"flash_mfma_bf16"
    info, _ = _info(heads=1, grid=(10, 15, 8), align=1, dtype=1, flags=_lib.FLAG_REFINE)
    assert L.monarch_attn_kernel_name(info.stage2_kernel) == b"generic_valu_fp32"
    info, _ = _info(heads=1, grid=(10, 15, 8), align=1, flags=_lib.FLAG_REFINE | _lib.FLAG_GENERIC)
    assert L.monarch_attn_kernel_name(info.stage2_kernel) == b"generic_valu_fp32"


def test_refine_unsupported_entry_points():
    st, h = _plan(heads=2, grid=(4, 6, 10), flags=_lib.FLAG_REFINE)
    assert st == _lib.OK
    assert L.monarch_attn_stage2(h, A, A + STEP, A + 2 * STEP, A + 3 * STEP, None) == _lib.ERR_UNSUPPORTED
    assert L.monarch_attn_chunk_forward(h, 0, 2, A, A + STEP, A + 2 * STEP, A + 3 * STEP, A + 4 * STEP,
                                        None) == _lib.ERR_UNSUPPORTED
    assert L.monarch_attn_backward_workspace_size(h) == 0
    assert L.monarch_attn_forward_train(h, A, A + STEP, A + 2 * STEP, A + 3 * STEP, A + 4 * STEP, 1 << 30,
                                        None) == _lib.ERR_UNSUPPORTED
    # the forward checks the larger workspace
    ws = L.monarch_attn_workspace_size(h)
    assert _fwd(h, ws_n=ws - 1) == _lib.ERR_WORKSPACE
    L.monarch_attn_destroy(h)


def test_fused_error_offset():
    info, ws = _info(heads=12, grid=(21, 30, 52), flags=_lib.FLAG_FUSED)
    y = 12 * 32760 * 128 * 2
    assert info.fused == 1 and info.fused_error_offset == (y + 255) // 256 * 256 + 16 * 4
    assert info.fused_error_offset + 4 <= ws
