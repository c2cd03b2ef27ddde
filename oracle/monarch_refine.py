"""fp64 CPU oracle of the refined Monarch factors (one or more refinement steps).

TEST INFRASTRUCTURE ONLY, like the rest of ``oracle/``: the product path never
imports, calls or links it. It shares no code with the HIP path.

What the pages say: the original MonarchAttention fits the Monarch factors
by iterative refinement and needs about ten steps; MonarchRT finetunes the
model so that a single refinement step at inference matches the quality of
the ten-step fit (gist.science English explainer, section 2.C "Finetuning and
Efficient Implementation"; Spanish explainer, Resumen Ejecutivo, section 2,
Metodologia B, "Reduccion de Costo de Inferencia"). The pages give no update
equations. The reading this oracle fixes (every step below is derived here,
not taken from the pages):

* Softmax attention is the maximiser of an entropy-regularised objective:
  for logits z_r of row r, softmax(z_r) is the unique maximiser over the
  probability simplex of <a, z_r> + H(a), H the Shannon entropy in nats
  (Gibbs' variational principle). Over a whole row-stochastic matrix A with
  logits S = s*Q K^T the objective is F(A) = sum_r <A_r, S_r> + H(A_r).
* A refinement step maximises F over Monarch matrices, one factor at a time.
  Inside a tile the Monarch matrix is A[(i,j),(i',j')] = L_j[i,i'] *
  R_i'[j,j'] (L_j the stage-2 factor of in-block position j, R_i' the
  stage-1 factor of block i', both row-stochastic). Row (i,j) of A is the
  joint law of (i', j') with i' ~ L_j[i,:] and j' ~ R_i'[j,:] given i', so
  H(A_(i,j)) = H(L_j[i,:]) + sum_i' L_j[i,i'] H(R_i'[j,:]). Hence:
  - R given L: row j of R_i' maximises sum_i L_j[i,i'] (<R_i'[j,:], S_(i,j),(i',.)>
    + H(R_i'[j,:])), so R_i'[j,:] = softmax_j'(s <qbar_(i',j), K[i',j']>) with
    the mixed query qbar_(i',j) = sum_i L_j[i,i'] Q[i,j] / sum_i L_j[i,i'].
  - L given R: L_j[i,:] = softmax_i'(s <Q[i,j], kbar_(i',j)> + H(R_i'[j,:]))
    with the mixed key kbar_(i',j) = sum_j' R_i'[j,j'] K[i',j'] (the keys of
    block i' mixed by the stage-1 factor, as Y mixes the values).
* The iteration starts from L = identity and updates R first, then L. With
  L = identity the first R update is the stage-1 factor of the direct
  Monarch forward (mixed query = the query itself), so ONE refinement step is:
  stage 1 as in the direct forward (Y = R V), plus the mixed keys
  Kbar = R K and the entropies H(R_i'[j,:]); stage 2 takes its logits against
  Kbar with the entropy of each key's stage-1 row added. T steps repeat the
  pair of updates T times.

Each update is the exact maximiser given the other factor, so F never
decreases along the iteration, and F of any row-stochastic matrix is at most
F(softmax(S)) = sum_r logsumexp(S_r). The refined output is O = A V.

Parity against the authors' implementation is unpinned: the pages print no
equations, code or values for the refinement.
"""
from __future__ import annotations

import math
from typing import Optional

import numpy as np

from .monarch_oracle import _f64, _scale, _tau, check_plan, softmax_rows

__all__ = [
    "entropy_rows",
    "refine_factors",
    "monarch_refine_forward",
    "factors_matrix",
    "gibbs_objective",
    "monarch_direct_factors",
]


def entropy_rows(p: np.ndarray) -> np.ndarray:
    """Shannon entropy (nats) of each row of a row-stochastic array, 0 log 0 = 0."""
    p = np.asarray(p, dtype=np.float64)
    with np.errstate(divide="ignore", invalid="ignore"):
        t = np.where(p > 0, p * np.log(p), 0.0)
    return -t.sum(axis=-1)


def _groups(x: np.ndarray, U: int, mt: int, b: int) -> np.ndarray:
    """[N, d] -> [U, m_tau, b, d]: tile u, block i, in-block position j."""
    return x.reshape(U, mt, b, x.shape[-1])


def _update_r(qt, kt, L, s):
    """Stage-1 factors given the stage-2 factors (one tile batch).

    qt, kt: [U, m, b, d]; L: [U, b, m, m] (group j: rows i, cols i').
    Returns R [U, m, b, b] (block i': rows j, cols j')."""
    w = L.transpose(0, 3, 1, 2)                  # [U, i', j, i] = L_j[i, i']
    col = w.sum(axis=-1, keepdims=True)          # [U, i', j, 1]
    qbar = np.einsum("uaji,uijd->uajd", w, qt) / col   # mixed queries [U, i', j, d]
    return softmax_rows(s * np.matmul(qbar, kt.transpose(0, 1, 3, 2)))


def _update_l(qt, kt, R, s):
    """Stage-2 factors given the stage-1 factors (one tile batch).

    Returns L [U, b, m, m] and the per-(i', j) entropies [U, m, b]."""
    kbar = np.matmul(R, kt)                      # [U, i', j, d]: keys of block i' mixed by R
    ent = entropy_rows(R)                        # [U, i', j]
    qg = qt.transpose(0, 2, 1, 3)                # [U, j, i, d]
    kg = kbar.transpose(0, 2, 1, 3)              # [U, j, i', d]
    z = s * np.matmul(qg, kg.transpose(0, 1, 3, 2)) + ent.transpose(0, 2, 1)[:, :, None, :]
    return softmax_rows(z), ent


def refine_factors(q, k, b: int, tile_tokens: Optional[int] = None, scale: Optional[float] = None,
                   steps: int = 1):
    """Monarch factors of one head after `steps` refinement steps (q, k: [N, d]).

    Returns (L, R): L [U, b, m_tau, m_tau] with L[u, j, i, i'] the stage-2 weight of
    block i' for the query at (i, j) of tile u; R [U, m_tau, b, b] with R[u, i', j, j']
    the stage-1 weight of position j' for row (i', j). steps = 0 returns L = identity and
    R from the first update's starting point is not formed (R = None)."""
    q, k = _f64(q), _f64(k)
    N, d = q.shape
    tau = _tau(N, tile_tokens)
    check_plan(N, b, tau)
    s = _scale(d, scale)
    U, mt = N // tau, tau // b
    qt, kt = _groups(q, U, mt, b), _groups(k, U, mt, b)
    L = np.broadcast_to(np.eye(mt), (U, b, mt, mt)).copy()
    R = None
    for _ in range(int(steps)):
        R = _update_r(qt, kt, L, s)
        L, _ = _update_l(qt, kt, R, s)
    return L, R


def monarch_refine_forward(q, k, v, b: int, tile_tokens: Optional[int] = None,
                           scale: Optional[float] = None, steps: int = 1,
                           return_parts: bool = False):
    """O = A V with A the Monarch matrix after `steps` (>= 1) refinement steps.

    Inputs [..., N, d] (leading dims looped). With return_parts=True (one head,
    inputs [N, d]) also returns the last step's mixed keys Kbar [N, d], the
    stage-1 entropies in nats [N] and Y = R V [N, d]."""
    if steps < 1:
        raise ValueError("at least one refinement step")
    q, k, v = _f64(q), _f64(k), _f64(v)
    *lead, N, d = q.shape
    tau = _tau(N, tile_tokens)
    check_plan(N, b, tau)
    s = _scale(d, scale)
    U, mt = N // tau, tau // b
    qf, kf, vf = q.reshape(-1, N, d), k.reshape(-1, N, d), v.reshape(-1, N, d)
    out = np.empty_like(qf)
    parts = None
    for h in range(qf.shape[0]):
        qt, kt, vt = _groups(qf[h], U, mt, b), _groups(kf[h], U, mt, b), _groups(vf[h], U, mt, b)
        L = np.broadcast_to(np.eye(mt), (U, b, mt, mt)).copy()
        for _ in range(int(steps)):
            R = _update_r(qt, kt, L, s)
            L, ent = _update_l(qt, kt, R, s)
        y = np.matmul(R, vt)                               # [U, i', j, d] stage 1
        og = np.matmul(L, y.transpose(0, 2, 1, 3))         # [U, j, i, d] stage 2
        out[h] = og.transpose(0, 2, 1, 3).reshape(N, d)
        if return_parts:
            parts = (np.matmul(R, kt).reshape(N, d), ent.reshape(N), y.reshape(N, d))
    out = out.reshape(*lead, N, d)
    return (out, parts) if return_parts else out


def monarch_direct_factors(q, k, b: int, tile_tokens: Optional[int] = None,
                           scale: Optional[float] = None):
    """The factors of the direct (unrefined) Monarch forward, in the layouts of
    ``refine_factors``: R from raw logits inside each block, L from raw logits
    inside each group."""
    q, k = _f64(q), _f64(k)
    N, d = q.shape
    tau = _tau(N, tile_tokens)
    check_plan(N, b, tau)
    s = _scale(d, scale)
    U, mt = N // tau, tau // b
    qt, kt = _groups(q, U, mt, b), _groups(k, U, mt, b)
    R = softmax_rows(s * np.matmul(qt, kt.transpose(0, 1, 3, 2)))
    qg, kg = qt.transpose(0, 2, 1, 3), kt.transpose(0, 2, 1, 3)
    L = softmax_rows(s * np.matmul(qg, kg.transpose(0, 1, 3, 2)))
    return L, R


def factors_matrix(L: np.ndarray, R: np.ndarray) -> np.ndarray:
    """The explicit N x N matrix A[(u,i,j),(u,i',j')] = L[u,j,i,i'] * R[u,i',j,j'],
    entry by entry with Python loops (tiny inputs only)."""
    U, b, mt, _ = L.shape
    tau = mt * b
    N = U * tau
    A = np.zeros((N, N))
    for u in range(U):
        for i in range(mt):
            for j in range(b):
                row = u * tau + i * b + j
                for i2 in range(mt):
                    for j2 in range(b):
                        A[row, u * tau + i2 * b + j2] = L[u, j, i, i2] * R[u, i2, j, j2]
    return A


def gibbs_objective(A: np.ndarray, q, k, scale: Optional[float] = None) -> float:
    """F(A) = sum over rows of <A_r, S_r> + H(A_r), S = s Q K^T, for an explicit
    row-stochastic N x N matrix A, entry by entry (0 log 0 = 0)."""
    q, k = _f64(q), _f64(k)
    N, d = q.shape
    s = _scale(d, scale)
    S = s * (q @ k.T)
    tot = 0.0
    for r in range(N):
        for c in range(N):
            a = A[r, c]
            if a > 0:
                tot += a * S[r, c] - a * math.log(a)
    return tot
