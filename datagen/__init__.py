"""Seeded synthetic inputs for Monarch video attention.

This module is the only code shared by the CPU oracle and the HIP path's
tests and bench. It draws Q, K, V tensors; it holds none of the attention
arithmetic itself (no logits, no softmax, no block or group mapping).

Token order on the video grid is (t, h, w) row-major, frame outermost:
n = (t*H + h)*W + w.

Distributions (the pages only say that video attention carries a pronounced
periodic structure driven by spatiotemporal position -- MonarchRT abstract;
gist.science explainer, "Problem Statement"):

* ``qkv``: X = N(0,1) + pe_scale * PE(t,h,w) for X in {Q, K, V}; one PE shared
  by Q, K, V, every batch and every head. PE is a per-axis sinusoidal code
  with the channel split (d_t, d_h, d_w) = (d - 4*floor(d/6), 2*floor(d/6),
  2*floor(d/6)); for an axis with d_a channels and position p the first half
  holds sin(p*w_k), the second half cos(p*w_k), w_k = 10000**(-2k/d_a).
* ``separable_qkv``: Q and K rows are concatenations [a_t ; c_h ; e_w] of
  per-axis tables drawn iid N(0,1) with the same channel split, so that a
  query/key logit is a sum of one term per axis (the separable positional
  component the pages describe as exactly preserved by aligned blocks).
  V is iid N(0,1).
* ``noisy_separable_qkv``: the separable Q and K plus noise * N(0,1) per
  element (a separate seeded draw); noise sets how far the logits are from
  separable (0 = exactly separable).

The normal draws are fp32 from a seeded ``torch.Generator`` on the CPU; the
result is cast to the requested dtype (round-to-nearest-even for bf16). The
oracle upcasts the very same tensors, so input quantisation never enters a
comparison.
"""
from __future__ import annotations

from typing import Sequence, Tuple

import numpy as np
import torch

__all__ = [
    "axis_channels",
    "positional_code",
    "qkv",
    "separable_qkv",
    "iid_qkv",
    "noisy_separable_qkv",
    "CONFIGS",
    "config_inputs",
]


def axis_channels(d: int) -> Tuple[int, int, int]:
    """Channel split (d_t, d_h, d_w) of a d-wide head; each part is even."""
    s = d // 6
    dt, dh, dw = d - 4 * s, 2 * s, 2 * s
    if min(dt, dh, dw) <= 0 or dt % 2 or dh % 2 or dw % 2:
        raise ValueError(f"head_dim {d} too small for a 3-axis code")
    return dt, dh, dw


def _axis_code(n_pos: int, width: int) -> np.ndarray:
    half = width // 2
    k = np.arange(half, dtype=np.float64)
    omega = 10000.0 ** (-2.0 * k / width)
    p = np.arange(n_pos, dtype=np.float64)[:, None]
    return np.concatenate([np.sin(p * omega), np.cos(p * omega)], axis=1)


def positional_code(T: int, H: int, W: int, d: int) -> np.ndarray:
    """[T*H*W, d] float64 sinusoidal (t, h, w) code, rows in (t, h, w) order."""
    dt, dh, dw = axis_channels(d)
    ct, ch, cw = _axis_code(T, dt), _axis_code(H, dh), _axis_code(W, dw)
    t = np.repeat(np.arange(T), H * W)
    h = np.tile(np.repeat(np.arange(H), W), T)
    w = np.tile(np.arange(W), T * H)
    return np.concatenate([ct[t], ch[h], cw[w]], axis=1)


def _randn(shape: Sequence[int], seed: int) -> torch.Tensor:
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    return torch.randn(tuple(shape), generator=g, dtype=torch.float32)


def qkv(batch: int, heads: int, grid: Tuple[int, int, int], d: int,
        seeds: Tuple[int, int, int], dtype: torch.dtype = torch.bfloat16,
        pe_scale: float = 0.5):
    """Q, K, V of shape [batch, heads, N, d] on the CPU in ``dtype``."""
    T, H, W = grid
    N = T * H * W
    pe = torch.from_numpy(pe_scale * positional_code(T, H, W, d)).to(torch.float32)
    out = []
    for s in seeds:
        x = _randn((batch, heads, N, d), s)
        if pe_scale:
            x += pe
        out.append(x.to(dtype).contiguous())
    return tuple(out)


def iid_qkv(batch: int, heads: int, N: int, d: int,
            seeds: Tuple[int, int, int], dtype: torch.dtype = torch.float32):
    """Q, K, V iid N(0,1), shape [batch, heads, N, d]."""
    return tuple(_randn((batch, heads, N, d), s).to(dtype).contiguous() for s in seeds)


def separable_qkv(batch: int, heads: int, grid: Tuple[int, int, int], d: int,
                  seed: int, dtype: torch.dtype = torch.bfloat16):
    """Q, K with per-axis separable rows [a_t; c_h; e_w]; V iid N(0,1)."""
    T, H, W = grid
    N = T * H * W
    dt, dh, dw = axis_channels(d)
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))

    def draw(*shape):
        return torch.randn(shape, generator=g, dtype=torch.float32)

    t = torch.arange(T).repeat_interleave(H * W)
    h = torch.arange(H).repeat_interleave(W).repeat(T)
    w = torch.arange(W).repeat(T * H)
    mats = []
    for _ in range(2):  # Q then K
        a, c, e = draw(batch, heads, T, dt), draw(batch, heads, H, dh), draw(batch, heads, W, dw)
        mats.append(torch.cat([a[:, :, t], c[:, :, h], e[:, :, w]], dim=-1).to(dtype).contiguous())
    v = draw(batch, heads, N, d).to(dtype).contiguous()
    return mats[0], mats[1], v


# The five workloads: name -> shape, dtype, alignment, tile and seeds.
CONFIGS = {
    "tiny_fp32": dict(batch=1, heads=1, d=64, grid=(8, 8, 8), align="frame", tile_tokens=0,
                      dtype="fp32", seeds=(0, 1, 2), pe_scale=0.0),
    "frame_bf16": dict(batch=1, heads=12, d=128, grid=(21, 30, 52), align="frame", tile_tokens=0,
                       dtype="bf16", seeds=(1000, 1001, 1002), pe_scale=0.5),
    "row_bf16": dict(batch=1, heads=12, d=128, grid=(21, 30, 52), align="row", tile_tokens=0,
                     dtype="bf16", seeds=(1000, 1001, 1002), pe_scale=0.5),
    "tiled_bf16": dict(batch=1, heads=12, d=128, grid=(21, 30, 52), align="frame", tile_tokens=4680,
                       dtype="bf16", seeds=(1000, 1001, 1002), pe_scale=0.5),
    "long_bf16": dict(batch=1, heads=12, d=128, grid=(81, 30, 52), align="frame", tile_tokens=0,
                      dtype="bf16", seeds=(2000, 2001, 2002), pe_scale=0.5),
}


def noisy_separable_qkv(batch: int, heads: int, grid: Tuple[int, int, int], d: int,
                        seed: int, noise: float, dtype: torch.dtype = torch.bfloat16):
    """separable_qkv (drawn in fp32) plus noise * N(0,1) on Q and K (seed + 1, + 2)."""
    q, k, v = separable_qkv(batch, heads, grid, d, seed, dtype=torch.float32)
    if noise:
        q = q + noise * _randn(q.shape, seed + 1)
        k = k + noise * _randn(k.shape, seed + 2)
    return tuple(x.to(dtype).contiguous() for x in (q, k, v))


def torch_dtype(name: str) -> torch.dtype:
    return {"bf16": torch.bfloat16, "fp32": torch.float32}[name]


def config_inputs(name: str, heads: int | None = None):
    """CPU Q, K, V for one of the named workloads (optionally fewer heads)."""
    c = CONFIGS[name]
    hh = c["heads"] if heads is None else heads
    if c["pe_scale"] == 0.0:
        T, H, W = c["grid"]
        return iid_qkv(c["batch"], hh, T * H * W, c["d"], c["seeds"], torch_dtype(c["dtype"]))
    return qkv(c["batch"], hh, c["grid"], c["d"], c["seeds"], torch_dtype(c["dtype"]), c["pe_scale"])
