"""Python binding of the Monarch video-attention library.

Marshals torch device tensors into the C ABI of include/monarch_attn.h and
launches on torch's current HIP stream. PyTorch supplies device memory and
streams only: every step of the computation runs in the library's kernels.
Tensors must live on a GPU; there is no CPU path.
"""
from __future__ import annotations

import ctypes
from typing import Optional, Sequence

import torch

from . import _lib

_DTYPES = {torch.bfloat16: _lib.BF16, torch.float32: _lib.FP32}
_DTYPE_NAMES = {"bf16": torch.bfloat16, "fp32": torch.float32}


class MonarchError(RuntimeError):
    def __init__(self, status: int, where: str):
        msg = _lib.lib().monarch_status_string(status).decode()
        super().__init__(f"{where}: {_lib.STATUS_NAMES.get(status, status)} ({msg})")
        self.status = status


def _check(status: int, where: str) -> None:
    if status != _lib.OK:
        raise MonarchError(status, where)


class MonarchPlan:
    """A validated problem: grid, alignment, tile, dtype (host metadata only).

    align: "frame" (b = H*W), "row" (b = W), "dense" (b = N), "token" (b = 1)
    or "custom" (b = custom_b). tile_tokens: 0/None = untiled. dtype: torch
    dtype or "bf16"/"fp32". refine: one refinement step of the factors
    (MONARCH_FLAG_REFINE).
    """

    def __init__(self, batch: int, heads: int, head_dim: int, grid: Sequence[int],
                 align: str = "frame", custom_b: int = 0, tile_tokens: Optional[int] = None,
                 dtype=torch.bfloat16, scale: Optional[float] = None, y_fp32: bool = False,
                 allow_unaligned: bool = False, generic: bool = False, fused: bool = False,
                 refine: bool = False):
        L = _lib.lib()
        if isinstance(dtype, str):
            dtype = _DTYPE_NAMES[dtype]
        if dtype not in _DTYPES:
            raise ValueError(f"unsupported dtype {dtype}")
        self.dtype = dtype
        flags = ((_lib.FLAG_Y_FP32 if y_fp32 else 0) | (_lib.FLAG_ALLOW_UNALIGNED if allow_unaligned else 0)
                 | (_lib.FLAG_GENERIC if generic else 0) | (_lib.FLAG_FUSED if fused else 0)
                 | (_lib.FLAG_REFINE if refine else 0))
        T, H, W = (int(x) for x in grid)
        handle = ctypes.c_void_p()
        st = L.monarch_attn_plan(ctypes.byref(handle), batch, heads, head_dim, T, H, W,
                                 _lib.ALIGN[align], int(custom_b), int(tile_tokens or 0),
                                 _DTYPES[dtype], float(scale or 0.0), flags)
        _check(st, "monarch_attn_plan")
        self._h = handle
        info = _lib.PlanInfo()
        _check(L.monarch_attn_plan_info(self._h, ctypes.byref(info)), "monarch_attn_plan_info")
        self.info = info.as_dict()
        self.shape = (batch, heads, T * H * W, head_dim)
        self.y_dtype = torch.float32 if self.info["y_dtype"] == _lib.FP32 else torch.bfloat16

    # -- properties
    @property
    def workspace_bytes(self) -> int:
        return int(_lib.lib().monarch_attn_workspace_size(self._h))

    def kernel_names(self):
        """Kernels of stage 1 and stage 2 when run apart (monarch_attn_stage1/2)."""
        L = _lib.lib()
        return (L.monarch_attn_kernel_name(self.info["stage1_kernel"]).decode(),
                L.monarch_attn_kernel_name(self.info["stage2_kernel"]).decode())

    @property
    def fused(self) -> bool:
        """True when forward() makes one fused launch for both stages."""
        return bool(self.info["fused"])

    def fused_error(self, workspace: torch.Tensor) -> int:
        """Error word of a fused plan's control block after a forward (0 = none).

        Reads device memory (synchronises); for tests and diagnostics."""
        if not self.fused:
            return 0
        off = int(self.info["fused_error_offset"])
        return int(workspace[off:off + 4].view(torch.int32).item())

    @property
    def flops(self) -> int:
        return self.info["flops_stage1"] + self.info["flops_stage2"]

    # -- helpers
    def _check_io(self, *ts, dtype=None):
        """GPU, contiguous, the plan's shape and (default) the plan's element type: the
        C ABI takes bare pointers, so these checks are what bounds its reads and writes."""
        want = self.dtype if dtype is None else dtype
        for t in ts:
            if not isinstance(t, torch.Tensor) or not t.is_cuda:
                raise ValueError("tensors must be GPU tensors")
            if tuple(t.shape) != self.shape or not t.is_contiguous():
                raise ValueError(f"expected contiguous {self.shape}, got {tuple(t.shape)}")
            if t.dtype != want:
                raise ValueError(f"dtype {t.dtype} != expected {want}")

    @staticmethod
    def _check_workspace(ws):
        if not isinstance(ws, torch.Tensor) or not ws.is_cuda or not ws.is_contiguous():
            raise ValueError("the workspace must be a contiguous GPU tensor")

    @staticmethod
    def _stream(t: torch.Tensor):
        return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)

    def new_workspace(self, device) -> Optional[torch.Tensor]:
        n = self.workspace_bytes
        return torch.empty(n, dtype=torch.uint8, device=device) if n else None

    # -- entry points
    def forward(self, q, k, v, out=None, workspace=None):
        self._check_io(q, k, v)
        if out is None:
            out = torch.empty_like(q)
        self._check_io(out)
        if workspace is None:
            workspace = self.new_workspace(q.device)
        if workspace is not None:
            self._check_workspace(workspace)
        ws_ptr = workspace.data_ptr() if workspace is not None else None
        ws_n = workspace.numel() * workspace.element_size() if workspace is not None else 0
        st = _lib.lib().monarch_attn_forward(self._h, q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                             out.data_ptr(), ws_ptr, ws_n, self._stream(q))
        _check(st, "monarch_attn_forward")
        return out

    def forward_noalloc(self, q, k, v, out):
        """forward() with the workspace taken from the library's static device array
        (monarch_attn_forward_noalloc): the library allocates nothing; `out` is required."""
        self._check_io(q, k, v, out)
        st = _lib.lib().monarch_attn_forward_noalloc(self._h, q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                                     out.data_ptr(), self._stream(q))
        _check(st, "monarch_attn_forward_noalloc")
        return out

    def stage1(self, q, k, v, y=None):
        self._check_io(q, k, v)
        ydt = self.y_dtype if self.info["m_tau"] > 1 else self.dtype
        if y is None:
            y = torch.empty(self.shape, dtype=ydt, device=q.device)
        self._check_io(y, dtype=ydt)
        st = _lib.lib().monarch_attn_stage1(self._h, q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                            y.data_ptr(), y.numel() * y.element_size(), self._stream(q))
        _check(st, "monarch_attn_stage1")
        return y

    def stage2(self, q, k, y, out=None):
        self._check_io(q, k)
        # Y has the plan's Y type, or the input type when stage 1 is the identity (b = 1: Y is V)
        self._check_io(y, dtype=self.y_dtype if self.info["b"] > 1 else self.dtype)
        if out is None:
            out = torch.empty_like(q)
        self._check_io(out)
        st = _lib.lib().monarch_attn_stage2(self._h, q.data_ptr(), k.data_ptr(), y.data_ptr(),
                                            out.data_ptr(), self._stream(q))
        _check(st, "monarch_attn_stage2")
        return out

    def chunk_forward(self, q, k, v, y, out, t0: int, t1: int):
        """Frames t0..t1-1 of frame-causal generation (see monarch_attn_chunk_forward).

        All tensors cover the whole video: reads q, v of the chunk, k of frames < t1
        and y (the stage-1 cache) of frames < t0; writes y and out of the chunk."""
        self._check_io(q, k, v, out)
        if y is not None:
            self._check_io(y, dtype=self.y_dtype)
        st = _lib.lib().monarch_attn_chunk_forward(self._h, int(t0), int(t1), q.data_ptr(), k.data_ptr(),
                                                   v.data_ptr(), y.data_ptr() if y is not None else None,
                                                   out.data_ptr(), self._stream(q))
        _check(st, "monarch_attn_chunk_forward")
        return out

    @property
    def backward_workspace_bytes(self) -> int:
        """Workspace bytes of backward() (0: this plan has no backward)."""
        return int(_lib.lib().monarch_attn_backward_workspace_size(self._h))

    def forward_train(self, q, k, v, out=None, workspace=None):
        """(O, workspace): O = forward(q, k, v), and a backward workspace holding the state
        backward(..., saved=True) uses instead of recomputing the forward."""
        self._check_io(q, k, v)
        if out is None:
            out = torch.empty_like(q)
        self._check_io(out)
        n = self.backward_workspace_bytes
        if workspace is None:
            workspace = torch.empty(max(n, 1), dtype=torch.uint8, device=q.device)
        self._check_workspace(workspace)
        ws_n = workspace.numel() * workspace.element_size()
        st = _lib.lib().monarch_attn_forward_train(self._h, q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                                   out.data_ptr(), workspace.data_ptr(), ws_n, self._stream(q))
        _check(st, "monarch_attn_forward_train")
        return out, workspace

    def backward(self, q, k, v, o, grad_o, workspace=None, grads=None, saved=False):
        """(dL/dQ, dL/dK, dL/dV) for O = forward(q, k, v) and grad_o = dL/dO.

        saved=True: `workspace` is the one forward_train(q, k, v) returned, unchanged since;
        the forward is then not recomputed."""
        if saved and workspace is None:
            raise ValueError("saved=True needs the workspace forward_train returned")
        self._check_io(q, k, v, o, grad_o)
        if grads is None:
            grads = tuple(torch.empty_like(q) for _ in range(3))
        self._check_io(*grads)
        n = self.backward_workspace_bytes
        if workspace is None:
            workspace = torch.empty(max(n, 1), dtype=torch.uint8, device=q.device)
        self._check_workspace(workspace)
        ws_n = workspace.numel() * workspace.element_size()
        fn = _lib.lib().monarch_attn_backward_saved if saved else _lib.lib().monarch_attn_backward
        st = fn(self._h, q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), grad_o.data_ptr(),
                grads[0].data_ptr(), grads[1].data_ptr(), grads[2].data_ptr(), workspace.data_ptr(), ws_n,
                self._stream(q))
        _check(st, "monarch_attn_backward_saved" if saved else "monarch_attn_backward")
        return grads

    def close(self):
        if getattr(self, "_h", None):
            _lib.lib().monarch_attn_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def monarch_attention(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, grid: Sequence[int],
                      align: str = "frame", tile_tokens: Optional[int] = None,
                      scale: Optional[float] = None, **kw) -> torch.Tensor:
    """Monarch attention of [B, Hh, N, d] GPU tensors over a (T, H, W) token grid."""
    B, Hh, N, d = q.shape
    plan = MonarchPlan(B, Hh, d, grid, align=align, tile_tokens=tile_tokens, dtype=q.dtype,
                       scale=scale, **kw)
    try:
        return plan.forward(q, k, v)
    finally:
        plan.close()
