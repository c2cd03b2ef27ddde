"""Monarch-factorized video attention on MI355X (gfx950).

The compute lives in libmonarch_attn.so (hand-written HIP kernels behind the
C ABI of include/monarch_attn.h); this package is its Python binding.
"""
from .attention import MonarchError, MonarchPlan, monarch_attention  # noqa: F401

__all__ = ["MonarchPlan", "MonarchError", "monarch_attention"]
