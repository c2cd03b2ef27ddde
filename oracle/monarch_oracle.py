"""fp64 CPU oracle for Monarch-factorized attention over a video token grid.

TEST INFRASTRUCTURE ONLY. This module exists to check the HIP library; the
product path never imports, calls or links it. Only ``tests/``,
``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` may use
it. It shares no code with the HIP path; the only common module is the
seeded input generator ``datagen``.

What is computed (sources are the MonarchRT pages: the author abstract as
reprinted on shd-paper.top and fugumt.com, and the gist.science English
explainer, section 2 "Methodology"):

* Attention over all N = T*H*W tokens of a video is replaced by a Monarch
  matrix: a product of two block-diagonal factors with a stride permutation
  between them (abstract; explainer section 2 intro).
* The blocks are aligned to the (frame, height, width) grid so that every
  video axis falls inside exactly one of the two block dimensions, e.g. block
  sizes (f*h, w) (explainer section 2.A "Block Alignment"). With tokens in
  (t, h, w) row-major order the aligned contiguous block sizes are b = H*W
  (one frame per block) and b = W (one spatial row per block).
* The tiled extension cuts each large block into smaller sub-blocks
  (explainer section 2.B "Tiled Monarch Parameterization"). Reading used
  here: the sequence is cut into tiles of tau tokens made of whole blocks;
  the Monarch product acts inside each tile and nothing crosses tiles.
* The attention is non-causal 3D attention (explainer section 2.C).

The pages never write the factor formulas. The spec reading this library
fixes, and this oracle follows:

  scale s = 1/sqrt(d) unless overridden.
  Tile u holds tokens u*tau .. u*tau+tau-1, m_tau = tau/b blocks per tile, and
  the token n = u*tau + i*b + j has block index i and in-block position j.
  Stage 1 (right factor, contiguous blocks): for every block,
      P1[j, j'] = softmax_j'( s * <Q[u,i,j], K[u,i,j']> ),
      Y[u,i,j]  = sum_j' P1[j, j'] * V[u,i,j'].
  Stage 2 (left factor, stride-b groups): for every tile u and position j,
      P2[i, i'] = softmax_i'( s * <Q[u,i,j], K[u,i',j]> ),
      O[u,i,j]  = sum_i' P2[i, i'] * Y[u,i',j].
  Matrix form: O = M V with M = P^T L P R, R = blockdiag of the P1 blocks,
  P the perfect-shuffle permutation (i, j) -> (j, i) inside each tile and
  L = blockdiag of the P2 groups; entrywise
      M[(u,i,j), (u,i',j')] = P2_{u,j}[i, i'] * P1_{u,i'}[j, j'].

All arithmetic is float64 with a max-subtracted softmax (stabilisation has no
effect in exact arithmetic). Inputs may be any float dtype; they are upcast.
"""
from __future__ import annotations

import math
from typing import Iterable, Optional, Sequence

import numpy as np

__all__ = [
    "block_size",
    "check_plan",
    "softmax_rows",
    "stage1",
    "stage2",
    "monarch_forward",
    "monarch_forward_groups",
    "monarch_matrix",
    "monarch_bruteforce",
    "dense_attention",
    "monarch_chunk_forward",
    "monarch_chunk_bruteforce",
    "flop_count",
]


# --------------------------------------------------------------------------
# plan arithmetic
# --------------------------------------------------------------------------
def block_size(grid: Sequence[int], align: str, custom_b: int = 0) -> int:
    """Block size b for an alignment on grid (T, H, W).

    frame: one frame per block, b = H*W (block dims (h*w, f), i.e. the pages'
    example (fh, w) family with the frame axis in the group dimension);
    row: one spatial row per block, b = W; dense: b = N (m = 1, ordinary
    attention); token: b = 1 (m = N, ordinary attention); custom: b as given.
    Explainer section 2.A "Block Alignment".
    """
    T, H, W = (int(x) for x in grid)
    N = T * H * W
    if align == "frame":
        return H * W
    if align == "row":
        return W
    if align == "dense":
        return N
    if align == "token":
        return 1
    if align == "custom":
        return int(custom_b)
    raise ValueError(f"unknown alignment {align!r}")


def check_plan(N: int, b: int, tau: int) -> None:
    """b must divide N; the tile tau must be whole blocks and divide N."""
    if b <= 0 or N % b:
        raise ValueError(f"block size {b} does not divide N={N}")
    if tau <= 0 or tau % b or N % tau:
        raise ValueError(f"tile {tau} must be a multiple of b={b} and divide N={N}")


def _tau(N: int, tile_tokens: Optional[int]) -> int:
    return N if not tile_tokens else int(tile_tokens)


def _scale(d: int, scale: Optional[float]) -> float:
    return 1.0 / math.sqrt(d) if not scale else float(scale)


def flop_count(batch: int, heads: int, N: int, d: int, b: int, m_tau: int) -> int:
    """Algorithmic FLOPs of one forward: QK^T and PV in both stages, 2 per MAC.

    Stage 1 does N*b logits and N*b value MACs per head, stage 2 does
    N*m_tau of each: 4*batch*heads*N*d*(b + m_tau).
    """
    return 4 * batch * heads * N * d * (b + m_tau)


# --------------------------------------------------------------------------
# the factored operator
# --------------------------------------------------------------------------
def softmax_rows(x: np.ndarray) -> np.ndarray:
    """Row softmax along the last axis, max-subtracted, float64."""
    x = np.asarray(x, dtype=np.float64)
    z = x - x.max(axis=-1, keepdims=True)
    e = np.exp(z)
    return e / e.sum(axis=-1, keepdims=True)


def _f64(a) -> np.ndarray:
    if hasattr(a, "detach"):  # torch tensor -> float64 numpy, exact upcast
        a = a.detach().to("cpu")
        import torch  # local: only needed for tensors
        a = a.to(torch.float64).numpy()
    return np.asarray(a, dtype=np.float64)


def stage1(q, k, v, b: int, scale: float) -> np.ndarray:
    """Right factor: softmax attention inside each contiguous block of b tokens.

    q, k, v: [N, d] float64. Returns Y [N, d].
    """
    N, d = q.shape
    nb = N // b
    qb, kb, vb = q.reshape(nb, b, d), k.reshape(nb, b, d), v.reshape(nb, b, d)
    logits = scale * np.matmul(qb, kb.transpose(0, 2, 1))  # [nb, b, b]
    p1 = softmax_rows(logits)
    return np.matmul(p1, vb).reshape(N, d)


def stage2(q, k, y, b: int, tau: int, scale: float) -> np.ndarray:
    """Left factor: softmax attention over each stride-b group inside a tile.

    The group of (tile u, position j) is the tokens u*tau + i*b + j,
    i = 0..tau/b-1. q, k, y: [N, d] float64. Returns O [N, d].
    """
    N, d = q.shape
    U, mt = N // tau, tau // b
    # [U, m_tau, b, d] -> [U, b, m_tau, d]: axis 2 of the result walks a group
    def groups(x):
        return x.reshape(U, mt, b, d).transpose(0, 2, 1, 3)

    qg, kg, yg = groups(q), groups(k), groups(y)
    logits = scale * np.matmul(qg, kg.transpose(0, 1, 3, 2))  # [U, b, m_tau, m_tau]
    p2 = softmax_rows(logits)
    og = np.matmul(p2, yg)  # [U, b, m_tau, d]
    return og.transpose(0, 2, 1, 3).reshape(N, d)


def monarch_forward(q, k, v, b: int, tile_tokens: Optional[int] = None,
                    scale: Optional[float] = None) -> np.ndarray:
    """O = stage2(stage1(V)) for inputs [..., N, d]; loops over leading dims."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    *lead, N, d = q.shape
    tau = _tau(N, tile_tokens)
    check_plan(N, b, tau)
    s = _scale(d, scale)
    qf, kf, vf = q.reshape(-1, N, d), k.reshape(-1, N, d), v.reshape(-1, N, d)
    out = np.empty_like(qf)
    for h in range(qf.shape[0]):
        y = stage1(qf[h], kf[h], vf[h], b, s)
        out[h] = stage2(qf[h], kf[h], y, b, tau, s)
    return out.reshape(*lead, N, d)


def monarch_forward_groups(q, k, v, b: int, tile_tokens: Optional[int],
                           scale: Optional[float], heads: Iterable[int],
                           groups: Iterable[tuple]) -> dict:
    """O on selected stage-2 groups only (for full-size sampled checks).

    q, k, v: [BH, N, d] (leading dims flattened). ``groups`` lists (u, j)
    pairs. Returns {(head, u, j): (token indices [m_tau], O rows [m_tau, d])}.
    Each Y row is computed from its own block exactly as in ``stage1``.
    """
    N, d = q.shape[-2:]
    tau = _tau(N, tile_tokens)
    check_plan(N, b, tau)
    s = _scale(d, scale)
    mt = tau // b
    res = {}
    for h in heads:
        qh, kh, vh = _f64(q[h]), _f64(k[h]), _f64(v[h])
        for (u, j) in groups:
            idx = u * tau + np.arange(mt) * b + j
            y = np.empty((mt, d))
            for r, n in enumerate(idx):
                blk = slice((n // b) * b, (n // b) * b + b)
                p1 = softmax_rows(s * (kh[blk] @ qh[n]))
                y[r] = p1 @ vh[blk]
            p2 = softmax_rows(s * (qh[idx] @ kh[idx].T))
            res[(h, u, j)] = (idx, p2 @ y)
    return res


# --------------------------------------------------------------------------
# explicit matrix forms (tiny inputs only)
# --------------------------------------------------------------------------
def monarch_matrix(q, k, b: int, tile_tokens: Optional[int] = None,
                   scale: Optional[float] = None) -> np.ndarray:
    """The N x N Monarch matrix M = P^T L P R for one head (q, k: [N, d]).

    Built from explicit factors: R block-diagonal over contiguous blocks,
    P the perfect shuffle inside each tile, L block-diagonal over the
    shuffled groups. Intended for N <= 2048.
    """
    q, k = _f64(q), _f64(k)
    N, d = q.shape
    tau = _tau(N, tile_tokens)
    check_plan(N, b, tau)
    s = _scale(d, scale)
    mt = tau // b
    R = np.zeros((N, N))
    for start in range(0, N, b):
        blk = slice(start, start + b)
        R[blk, blk] = softmax_rows(s * q[blk] @ k[blk].T)
    # P maps token (u, i, j) to shuffled slot (u, j, i): row slot, col token
    P = np.zeros((N, N))
    for u in range(N // tau):
        for i in range(mt):
            for j in range(b):
                P[u * tau + j * mt + i, u * tau + i * b + j] = 1.0
    qs, ks = P @ q, P @ k  # shuffled order: groups are contiguous runs of m_tau
    L = np.zeros((N, N))
    for start in range(0, N, mt):
        g = slice(start, start + mt)
        L[g, g] = softmax_rows(s * qs[g] @ ks[g].T)
    return P.T @ L @ P @ R


def monarch_bruteforce(q, k, v, b: int, tile_tokens: Optional[int] = None,
                       scale: Optional[float] = None) -> np.ndarray:
    """O from the entrywise definition with plain Python loops (N <= ~64).

    M[(u,i,j),(u,i',j')] = P2_{u,j}[i,i'] * P1_{u,i'}[j,j']; every weight is
    built from math.exp of the dot products, with no matrix library.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    N, d = q.shape
    tau = _tau(N, tile_tokens)
    check_plan(N, b, tau)
    s = _scale(d, scale)
    mt = tau // b

    def dot(a, c):
        return sum(float(a[e]) * float(c[e]) for e in range(d))

    def weights(row, cols):
        z = [s * dot(q[row], k[c]) for c in cols]
        top = max(z)
        ex = [math.exp(x - top) for x in z]
        tot = sum(ex)
        return [x / tot for x in ex]

    out = np.zeros((N, d))
    for u in range(N // tau):
        for i in range(mt):
            for j in range(b):
                n = u * tau + i * b + j
                group = [u * tau + i2 * b + j for i2 in range(mt)]
                p2 = weights(n, group)
                for i2 in range(mt):
                    n2 = group[i2]
                    block = [u * tau + i2 * b + j2 for j2 in range(b)]
                    p1 = weights(n2, block)
                    for j2 in range(b):
                        w = p2[i2] * p1[j2]
                        src = block[j2]
                        for e in range(d):
                            out[n, e] += w * float(v[src, e])
    return out


# --------------------------------------------------------------------------
# ordinary softmax attention (the dense comparison and special cases)
# --------------------------------------------------------------------------
def dense_attention(q, k, v, scale: Optional[float] = None,
                    rows: Optional[np.ndarray] = None,
                    key_tile: Optional[int] = None) -> np.ndarray:
    """softmax(s Q K^T) V for one head (q, k, v: [N, d]).

    ``rows``: compute only these query rows. ``key_tile``: restrict every
    query to keys in its own tile of that many tokens (tile-masked dense).
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    N, d = q.shape
    s = _scale(d, scale)
    rows = np.arange(N) if rows is None else np.asarray(rows)
    out = np.empty((len(rows), d))
    for c0 in range(0, len(rows), 1024):
        r = rows[c0:c0 + 1024]
        if key_tile:
            for idx, n in enumerate(r):
                t0 = (n // key_tile) * key_tile
                sl = slice(t0, t0 + key_tile)
                out[c0 + idx] = softmax_rows(s * (k[sl] @ q[n])) @ v[sl]
        else:
            out[c0:c0 + len(r)] = softmax_rows(s * (q[r] @ k.T)) @ v
    return out


def monarch_chunk_forward(q, k, v, b: int, frame_tokens: int, t0: int, t1: int,
                          scale: Optional[float] = None) -> np.ndarray:
    """One chunk of frame-causal generation: O for the frames t0..t1-1.

    The reading (the pages target autoregressive, chunk-by-chunk generation
    with Self-Forcing but give no formula for it): stage 1 is unchanged, its
    blocks lie inside frames; each stage-2 group keeps its rows of frames
    before t1 as keys and values and its rows of frames t0..t1-1 as queries.
    Inputs [..., N, d] over the whole video (untiled); rows of frames >= t1
    are never used. Returns O rows of the chunk, [..., (t1-t0)*frame_tokens, d].
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    *lead, N, d = q.shape
    check_plan(N, b, N)
    assert frame_tokens % b == 0 and N % frame_tokens == 0 and 0 <= t0 < t1 <= N // frame_tokens
    s = _scale(d, scale)
    bpf = frame_tokens // b
    r0, r1 = t0 * bpf, t1 * bpf  # block rows of the chunk, keys: blocks 0..r1-1
    qf, kf, vf = q.reshape(-1, N, d), k.reshape(-1, N, d), v.reshape(-1, N, d)
    out = np.empty((qf.shape[0], (r1 - r0) * b, d))
    for h in range(qf.shape[0]):
        n_keys = r1 * b  # tokens of frames 0..t1-1
        y = stage1(qf[h, :n_keys], kf[h, :n_keys], vf[h, :n_keys], b, s)  # [r1*b, d]
        qg = qf[h, :n_keys].reshape(r1, b, d).transpose(1, 0, 2)  # [b groups, r1 rows, d]
        kg = kf[h, :n_keys].reshape(r1, b, d).transpose(1, 0, 2)
        yg = y.reshape(r1, b, d).transpose(1, 0, 2)
        p2 = softmax_rows(s * np.matmul(qg[:, r0:r1], kg.transpose(0, 2, 1)))  # [b, r1-r0, r1]
        out[h] = np.matmul(p2, yg).transpose(1, 0, 2).reshape(-1, d)
    return out.reshape(*lead, (r1 - r0) * b, d)


def monarch_chunk_bruteforce(q, k, v, b: int, frame_tokens: int, t0: int, t1: int,
                             scale: Optional[float] = None) -> np.ndarray:
    """The chunk output by explicit loops over tokens (tiny inputs): for a
    query in block i (at in-block position j) of the chunk,
    O = sum_{i' < r1} P2[i, i'] * sum_j'' P1_{i'}[j, j''] * V[i' * b + j''],
    P2 normalised over the blocks i' < r1 only. q, k, v: [N, d]."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    N, d = q.shape
    s = _scale(d, scale)
    bpf = frame_tokens // b
    r0, r1 = t0 * bpf, t1 * bpf
    out = np.zeros(((r1 - r0) * b, d))
    for i in range(r0, r1):
        for j in range(b):
            n = i * b + j
            z2 = [s * float(np.dot(q[n], k[ip * b + j])) for ip in range(r1)]
            w2 = [math.exp(x - max(z2)) for x in z2]
            for ip in range(r1):
                p2 = w2[ip] / sum(w2)
                m = ip * b + j
                z1 = [s * float(np.dot(q[m], k[ip * b + jj])) for jj in range(b)]
                w1 = [math.exp(x - max(z1)) for x in z1]
                for jj in range(b):
                    out[n - r0 * b] += p2 * w1[jj] / sum(w1) * v[ip * b + jj]
    return out

