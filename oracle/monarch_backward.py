"""fp64 CPU oracle for the backward pass of Monarch attention.

TEST INFRASTRUCTURE ONLY, like ``monarch_oracle``: only ``tests/`` may import
it; the product path never does, and it shares no code with the HIP path.

What is computed: the gradients dL/dQ, dL/dK, dL/dV of a scalar loss L whose
gradient with respect to the forward output O is G (the pages ship forward
and backward kernels for fine-tuning, explainer section 2.C; they print no
formulas, so this is the chain rule applied to the forward spec in
``monarch_oracle``).

For one softmax-attention problem O = P V with P = rowsoftmax(s Q K^T):
  dV    = P^T G
  dP    = G V^T
  delta = rowsum(G * O)          (sum over channels, one value per row)
  dS    = P * (dP - delta)       (elementwise; the softmax Jacobian)
  dQ    = s dS K
  dK    = s dS^T Q
The Monarch operator is two such problems in sequence. Stage 2 (stride-b
groups, values Y = stage-1 output) turns G into dQ2, dK2 and dY; stage 1
(contiguous blocks, values V) turns dY into dQ1, dK1 and dV. Q and K feed
both stages, so dQ = dQ1 + dQ2 and dK = dK1 + dK2.
"""
from __future__ import annotations

from typing import Optional

import numpy as np

from .monarch_oracle import _f64, _scale, _tau, check_plan, softmax_rows, stage1

__all__ = ["attention_backward", "stage1_backward", "stage2_backward", "monarch_backward"]


def attention_backward(q, k, v, g, scale: float):
    """Gradients of O = rowsoftmax(scale * q k^T) v for upstream g.

    Batched over leading axes: q, k, v, g are [..., L, d] float64.
    Returns (dq, dk, dv), each [..., L, d].
    """
    kt = np.swapaxes(k, -1, -2)
    p = softmax_rows(scale * np.matmul(q, kt))
    o = np.matmul(p, v)
    dv = np.matmul(np.swapaxes(p, -1, -2), g)
    dp = np.matmul(g, np.swapaxes(v, -1, -2))
    delta = np.sum(g * o, axis=-1, keepdims=True)
    ds = p * (dp - delta)
    dq = scale * np.matmul(ds, k)
    dk = scale * np.matmul(np.swapaxes(ds, -1, -2), q)
    return dq, dk, dv


def stage1_backward(q, k, v, gy, b: int, scale: float):
    """Backward of the right factor (blocks of b contiguous tokens).

    q, k, v, gy: [N, d]. Returns (dq1, dk1, dv), each [N, d].
    """
    N, d = q.shape
    blk = lambda x: x.reshape(N // b, b, d)
    dq, dk, dv = attention_backward(blk(q), blk(k), blk(v), blk(gy), scale)
    return dq.reshape(N, d), dk.reshape(N, d), dv.reshape(N, d)


def stage2_backward(q, k, y, go, b: int, tau: int, scale: float):
    """Backward of the left factor (stride-b groups inside each tile).

    The group of (tile u, position j) is the tokens u*tau + i*b + j.
    q, k, y, go: [N, d]. Returns (dq2, dk2, dy), each [N, d].
    """
    N, d = q.shape
    U, mt = N // tau, tau // b

    def groups(x):
        return x.reshape(U, mt, b, d).transpose(0, 2, 1, 3)

    def ungroup(x):
        return x.transpose(0, 2, 1, 3).reshape(N, d)

    dq, dk, dy = attention_backward(groups(q), groups(k), groups(y), groups(go), scale)
    return ungroup(dq), ungroup(dk), ungroup(dy)


def monarch_backward(q, k, v, go, b: int, tile_tokens: Optional[int] = None,
                     scale: Optional[float] = None):
    """(dQ, dK, dV) of the Monarch forward for upstream gradient go.

    Inputs [..., N, d] of any float dtype (upcast exactly to float64); loops
    over the leading dims. Returns three float64 arrays of the input shape.
    """
    q, k, v, go = _f64(q), _f64(k), _f64(v), _f64(go)
    *lead, N, d = q.shape
    tau = _tau(N, tile_tokens)
    check_plan(N, b, tau)
    s = _scale(d, scale)
    flat = [x.reshape(-1, N, d) for x in (q, k, v, go)]
    dq, dk, dv = (np.empty_like(flat[0]) for _ in range(3))
    for h in range(flat[0].shape[0]):
        qh, kh, vh, gh = (x[h] for x in flat)
        y = stage1(qh, kh, vh, b, s)
        dq2, dk2, dy = stage2_backward(qh, kh, y, gh, b, tau, s)
        dq1, dk1, dv[h] = stage1_backward(qh, kh, vh, dy, b, s)
        dq[h] = dq1 + dq2
        dk[h] = dk1 + dk2
    return tuple(x.reshape(*lead, N, d) for x in (dq, dk, dv))
