"""ctypes declarations of the C ABI in include/monarch_attn.h.

Argument marshalling only: no arithmetic of the method happens here. The
library is loaded from this package directory; if it is missing the import of
any entry point raises, there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
# always the in-tree build (structured_attention_video_amd/build.py writes it)
LIB_PATH = os.path.join(_HERE, "libmonarch_attn.so")

# status codes (monarch_status)
OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_UNALIGNED, ERR_WORKSPACE, ERR_ALIAS, ERR_HIP, ERR_TOO_LARGE = range(8)
STATUS_NAMES = {
    OK: "MONARCH_OK", ERR_INVALID_ARG: "MONARCH_ERR_INVALID_ARG",
    ERR_UNSUPPORTED: "MONARCH_ERR_UNSUPPORTED", ERR_UNALIGNED: "MONARCH_ERR_UNALIGNED",
    ERR_WORKSPACE: "MONARCH_ERR_WORKSPACE", ERR_ALIAS: "MONARCH_ERR_ALIAS", ERR_HIP: "MONARCH_ERR_HIP",
    ERR_TOO_LARGE: "MONARCH_ERR_TOO_LARGE",
}
# bytes of the static device array monarch_attn_forward_noalloc works in (MONARCH_NOALLOC_SCRATCH_BYTES)
NOALLOC_SCRATCH_BYTES = 128 << 20
# monarch_dtype
BF16, FP32 = 0, 1
# monarch_align
ALIGN = {"frame": 0, "row": 1, "dense": 2, "token": 3, "custom": 4}
# flags
FLAG_Y_FP32, FLAG_ALLOW_UNALIGNED, FLAG_GENERIC, FLAG_FUSED, FLAG_REFINE = 1, 2, 4, 8, 16

EXPORTED = [
    "monarch_attn_plan", "monarch_attn_destroy", "monarch_attn_workspace_size",
    "monarch_attn_plan_info", "monarch_attn_forward", "monarch_attn_stage1",
    "monarch_attn_stage2", "monarch_status_string", "monarch_attn_kernel_name",
    "monarch_attn_abi_version", "monarch_attn_backward_workspace_size", "monarch_attn_backward",
    "monarch_attn_chunk_forward", "monarch_attn_forward_train", "monarch_attn_backward_saved",
    "monarch_attn_forward_noalloc",
]


class PlanInfo(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int64), ("heads", ctypes.c_int64), ("head_dim", ctypes.c_int64),
        ("T", ctypes.c_int64), ("H", ctypes.c_int64), ("W", ctypes.c_int64), ("N", ctypes.c_int64),
        ("b", ctypes.c_int64), ("tau", ctypes.c_int64), ("m_tau", ctypes.c_int64),
        ("tiles", ctypes.c_int64), ("dtype", ctypes.c_int32), ("y_dtype", ctypes.c_int32),
        ("scale", ctypes.c_float), ("flags", ctypes.c_uint32), ("workspace_bytes", ctypes.c_int64),
        ("flops_stage1", ctypes.c_int64), ("flops_stage2", ctypes.c_int64),
        ("stage1_kernel", ctypes.c_int32), ("stage2_kernel", ctypes.c_int32), ("fused", ctypes.c_int32),
        ("refine_steps", ctypes.c_int32), ("fused_error_offset", ctypes.c_int64),
    ]

    def as_dict(self):
        return {name: getattr(self, name) for name, _ in self._fields_}


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is missing: build the HIP library first "
            "(python -m structured_attention_video_amd.build)")
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, f32, u32, sz = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64,
                                  ctypes.c_float, ctypes.c_uint32, ctypes.c_size_t)
    L.monarch_attn_plan.argtypes = [ctypes.POINTER(vp), i32, i32, i32, i32, i32, i32, i32, i64, i64,
                                    i32, f32, u32]
    L.monarch_attn_plan.restype = i32
    L.monarch_attn_destroy.argtypes = [vp]
    L.monarch_attn_destroy.restype = None
    L.monarch_attn_workspace_size.argtypes = [vp]
    L.monarch_attn_workspace_size.restype = sz
    L.monarch_attn_plan_info.argtypes = [vp, ctypes.POINTER(PlanInfo)]
    L.monarch_attn_plan_info.restype = i32
    L.monarch_attn_forward.argtypes = [vp, vp, vp, vp, vp, vp, sz, vp]
    L.monarch_attn_forward.restype = i32
    L.monarch_attn_stage1.argtypes = [vp, vp, vp, vp, vp, sz, vp]
    L.monarch_attn_stage1.restype = i32
    L.monarch_attn_stage2.argtypes = [vp, vp, vp, vp, vp, vp]
    L.monarch_attn_stage2.restype = i32
    L.monarch_status_string.argtypes = [i32]
    L.monarch_status_string.restype = ctypes.c_char_p
    L.monarch_attn_kernel_name.argtypes = [i32]
    L.monarch_attn_kernel_name.restype = ctypes.c_char_p
    L.monarch_attn_abi_version.argtypes = []
    L.monarch_attn_abi_version.restype = i32
    L.monarch_attn_backward_workspace_size.argtypes = [vp]
    L.monarch_attn_backward_workspace_size.restype = sz
    L.monarch_attn_backward.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    L.monarch_attn_backward.restype = i32
    L.monarch_attn_chunk_forward.argtypes = [vp, i32, i32, vp, vp, vp, vp, vp, vp]
    L.monarch_attn_chunk_forward.restype = i32
    L.monarch_attn_forward_train.argtypes = [vp, vp, vp, vp, vp, vp, sz, vp]
    L.monarch_attn_forward_train.restype = i32
    L.monarch_attn_backward_saved.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    L.monarch_attn_backward_saved.restype = i32
    L.monarch_attn_forward_noalloc.argtypes = [vp, vp, vp, vp, vp, vp]
    L.monarch_attn_forward_noalloc.restype = i32
    _lib = L
    return L
