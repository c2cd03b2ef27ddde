"""Pins of the refinement-step oracle (oracle/monarch_refine.py) that do not
reuse its formulas: library attention for the degenerate block sizes, the
exactness the pages claim for aligned blocks on separable logits, the
variational objective evaluated entry by entry on explicit N x N matrices
(its chain of inequalities and the first-order optimality of each update,
by finite differences), closed forms, and planted mistakes that must fail.
"""
import math

import numpy as np
import pytest
import torch

import datagen
import oracle
from oracle import monarch_refine as mr


def _rand(shape, seed, scale=1.0):
    return scale * np.random.default_rng(seed).standard_normal(shape)


def _sdpa(q, k, v, mask=None, scale=None):
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a))[None]
    return torch.nn.functional.scaled_dot_product_attention(
        t(q), t(k), t(v), attn_mask=None if mask is None else torch.from_numpy(mask)[None],
        scale=scale)[0].numpy()


def _logsumexp_rows(x):
    m = x.max(axis=1, keepdims=True)
    return (m[:, 0] + np.log(np.exp(x - m).sum(axis=1)))


# ---------------------------------------------------------------- degenerate block sizes
@pytest.mark.parametrize("b", [40, 1])
@pytest.mark.parametrize("steps", [1, 3])
def test_dense_special_cases_match_library(b, steps):
    N, d = 40, 8
    q, k, v = _rand((N, d), 1), _rand((N, d), 2), _rand((N, d), 3)
    got = mr.monarch_refine_forward(q, k, v, b, steps=steps)
    np.testing.assert_allclose(got, _sdpa(q, k, v), atol=1e-13)


def test_tile_equal_block_is_block_diagonal_attention():
    N, d, b = 36, 6, 12
    q, k, v = _rand((N, d), 4), _rand((N, d), 5), _rand((N, d), 6)
    blk = np.arange(N) // b
    got = mr.monarch_refine_forward(q, k, v, b, b, steps=2)
    np.testing.assert_allclose(got, _sdpa(q, k, v, blk[:, None] == blk[None, :]), atol=1e-13)


# ---------------------------------------------------------------- separable logits (aligned exactness)
GRID = (3, 4, 5)


def _sep(d=12, seed=17):
    q, k, v = datagen.separable_qkv(1, 1, GRID, d, seed, dtype=torch.float64)
    return q[0, 0].numpy(), k[0, 0].numpy(), v[0, 0].numpy()


@pytest.mark.parametrize("align", ["frame", "row"])
@pytest.mark.parametrize("steps", [1, 2])
def test_separable_exact_when_aligned(align, steps):
    q, k, v = _sep()
    b = oracle.block_size(GRID, align)
    got = mr.monarch_refine_forward(q, k, v, b, steps=steps)
    np.testing.assert_allclose(got, oracle.dense_attention(q, k, v), atol=1e-12)


def test_separable_tiled_equals_tile_masked_dense():
    q, k, v = _sep()
    T, H, W = GRID
    got = mr.monarch_refine_forward(q, k, v, W, H * W)
    np.testing.assert_allclose(got, oracle.dense_attention(q, k, v, key_tile=H * W), atol=1e-12)


def test_misaligned_split_not_exact():
    q, k, v = _sep()
    T, H, W = GRID
    err = np.abs(mr.monarch_refine_forward(q, k, v, 2 * W) - oracle.dense_attention(q, k, v)).max()
    assert err > 0.05, err


# ---------------------------------------------------------------- closed forms
@pytest.mark.parametrize("which", ["q", "k"])
def test_zero_logits_give_tile_mean(which):
    N, d = 24, 5
    q, k, v = _rand((N, d), 18), _rand((N, d), 19), _rand((N, d), 20)
    (q if which == "q" else k)[:] = 0
    for b, tau in [(6, None), (3, None), (6, 12)]:
        t = tau or N
        want = np.repeat(v.reshape(N // t, t, d).mean(axis=1), t, axis=0)
        np.testing.assert_allclose(mr.monarch_refine_forward(q, k, v, b, tau), want, atol=1e-14)


def test_constant_values_pass_through():
    N, d = 24, 5
    q, k = _rand((N, d), 21), _rand((N, d), 22)
    v = np.tile(_rand((1, d), 23), (N, 1))
    np.testing.assert_allclose(mr.monarch_refine_forward(q, k, v, 6, steps=2), v, atol=1e-14)


def test_entropy_rows_closed_forms():
    assert mr.entropy_rows(np.full((1, 8), 1 / 8))[0] == pytest.approx(math.log(8), abs=1e-15)
    assert mr.entropy_rows(np.eye(4)).tolist() == [0.0] * 4
    p = np.array([[0.5, 0.25, 0.25]])
    assert mr.entropy_rows(p)[0] == pytest.approx(1.5 * math.log(2), abs=1e-15)


# ---------------------------------------------------------------- explicit matrices and the objective
SMALL = [((4, 2, 3), 6, None), ((4, 2, 3), 3, None), ((4, 2, 3), 6, 12)]


@pytest.mark.parametrize("grid,b,tau", SMALL)
def test_factored_application_equals_explicit_matrix(grid, b, tau):
    N = int(np.prod(grid))
    q, k, v = _rand((N, 3), 30), _rand((N, 3), 31), _rand((N, 3), 32)
    for steps in (1, 2):
        L, R = mr.refine_factors(q, k, b, tau, steps=steps)
        A = mr.factors_matrix(L, R)
        np.testing.assert_allclose(A.sum(axis=1), 1.0, atol=1e-14)
        assert (A >= 0).all()
        t = tau or N
        blk = np.arange(N) // t
        assert (A[blk[:, None] != blk[None, :]] == 0).all()   # nothing crosses tiles
        np.testing.assert_allclose(A @ v, mr.monarch_refine_forward(q, k, v, b, tau, steps=steps),
                                   atol=1e-13)


def test_gibbs_objective_of_softmax_is_logsumexp():
    N, d = 12, 3
    q, k = _rand((N, d), 33), _rand((N, d), 34)
    S = (q @ k.T) / math.sqrt(d)
    A = oracle.softmax_rows(S)
    assert mr.gibbs_objective(A, q, k) == pytest.approx(_logsumexp_rows(S).sum(), abs=1e-12)
    # any other row-stochastic matrix is below it
    B = np.random.default_rng(35).dirichlet(np.ones(N), size=N)
    assert mr.gibbs_objective(B, q, k) < _logsumexp_rows(S).sum()


@pytest.mark.parametrize("grid,b,tau", SMALL)
def test_objective_increases_along_the_iteration(grid, b, tau):
    N = int(np.prod(grid))
    q, k = _rand((N, 3), 36, 1.5), _rand((N, 3), 37, 1.5)
    Ld, Rd = mr.monarch_direct_factors(q, k, b, tau)
    f = [mr.gibbs_objective(mr.factors_matrix(Ld, Rd), q, k)]
    for steps in (1, 2, 3, 6):
        L, R = mr.refine_factors(q, k, b, tau, steps=steps)
        f.append(mr.gibbs_objective(mr.factors_matrix(L, R), q, k))
    S = (q @ k.T) / math.sqrt(3)
    assert all(f[i] <= f[i + 1] + 1e-12 for i in range(len(f) - 1)), f
    t = tau or N
    # the upper bound: softmax inside each tile (Monarch rows never leave their tile)
    mask = (np.arange(N)[:, None] // t) == (np.arange(N)[None, :] // t)
    bound = _logsumexp_rows(np.where(mask, S, -np.inf)).sum()
    assert f[-1] <= bound + 1e-12
    assert f[1] > f[0] + 1e-6       # one step strictly improves on the direct factors here


def _objective(L, R, q, k):
    return mr.gibbs_objective(mr.factors_matrix(L, R), q, k)


def _step(x, a):
    """Finite-difference step along e_a - e_0 of one simplex row: small against both
    entries it moves (the objective's log terms curve on the scale of the entry)."""
    return 1e-3 * min(x[a], x[0], 1e-2)


def _kkt_gap_l(L, R, q, k):
    """Largest |dF/dL[.., a] - dF/dL[.., 0]| over every row of L (central finite
    differences of F on the explicit matrix): zero where L maximises F for this R."""
    U, b, mt, _ = L.shape
    gap = 0.0
    for u in range(U):
        for j in range(b):
            for i in range(mt):
                for a in range(1, mt):
                    h = _step(L[u, j, i], a)
                    Lp, Lm = L.copy(), L.copy()
                    Lp[u, j, i, a] += h; Lp[u, j, i, 0] -= h
                    Lm[u, j, i, a] -= h; Lm[u, j, i, 0] += h
                    g = (_objective(Lp, R, q, k) - _objective(Lm, R, q, k)) / (2 * h)
                    gap = max(gap, abs(g))
    return gap


def _kkt_gap_r(L, R, q, k):
    """As _kkt_gap_l for the rows of R with L fixed."""
    U, mt, b, _ = R.shape
    gap = 0.0
    for u in range(U):
        for i in range(mt):
            for j in range(b):
                for a in range(1, b):
                    h = _step(R[u, i, j], a)
                    Rp, Rm = R.copy(), R.copy()
                    Rp[u, i, j, a] += h; Rp[u, i, j, 0] -= h
                    Rm[u, i, j, a] -= h; Rm[u, i, j, 0] += h
                    g = (_objective(L, Rp, q, k) - _objective(L, Rm, q, k)) / (2 * h)
                    gap = max(gap, abs(g))
    return gap


KKT_CASE = ((2, 2, 3), 6, None)   # N = 12, frame blocks of 6, groups of 2
KKT_TOL = 1e-5


def _kkt_data():
    (T, H, W), b, tau = KKT_CASE
    N = T * H * W
    return _rand((N, 3), 50), _rand((N, 3), 51), b, tau


def test_each_update_satisfies_first_order_optimality():
    q, k, b, tau = _kkt_data()
    L1, R1 = mr.refine_factors(q, k, b, tau, steps=1)
    L2, R2 = mr.refine_factors(q, k, b, tau, steps=2)
    identity = np.broadcast_to(np.eye(L1.shape[-1]), L1.shape).copy()
    assert _kkt_gap_r(identity, R1, q, k) < KKT_TOL   # the first R update, L = identity
    assert _kkt_gap_l(L1, R1, q, k) < KKT_TOL          # L given R
    assert _kkt_gap_r(L1, R2, q, k) < KKT_TOL          # the second R update, given L of step 1
    assert _kkt_gap_l(L2, R2, q, k) < KKT_TOL
    # the direct factors are not a maximiser of either update (a nonzero gap)
    Ld, Rd = mr.monarch_direct_factors(q, k, b, tau)
    assert _kkt_gap_l(Ld, Rd, q, k) > 1e-3


def test_one_step_parts_are_the_direct_stage1():
    """One step from L = identity: Y is the direct forward's stage 1, the mixed keys are the
    direct stage-1 factor applied to K, the entropies are those of its rows."""
    N, d, b = 24, 4, 6
    q, k, v = _rand((N, d), 60), _rand((N, d), 61), _rand((N, d), 62)
    _, (kbar, ent, y) = mr.monarch_refine_forward(q, k, v, b, return_parts=True)
    s = 1 / math.sqrt(d)
    np.testing.assert_allclose(y, oracle.stage1(q, k, v, b, s), atol=1e-14)
    np.testing.assert_allclose(kbar, oracle.stage1(q, k, k, b, s), atol=1e-14)
    for n in range(N):
        blk = slice((n // b) * b, (n // b) * b + b)
        p = oracle.softmax_rows(s * (k[blk] @ q[n]))
        assert ent[n] == pytest.approx(-sum(x * math.log(x) for x in p), abs=1e-13)


# ---------------------------------------------------------------- planted mistakes
def _mutant_factors(q, k, b, tau, steps, mutation):
    """An independent copy of the alternating updates with one planted mistake."""
    N, d = q.shape
    tau = tau or N
    s = 1 / math.sqrt(d)
    U, mt = N // tau, tau // b
    qt, kt = q.reshape(U, mt, b, d), k.reshape(U, mt, b, d)
    sm = oracle.softmax_rows
    L = np.broadcast_to(np.eye(mt), (U, b, mt, mt)).copy()
    R = None
    for _ in range(steps):
        R = np.empty((U, mt, b, b))
        for u in range(U):
            for ip in range(mt):
                for j in range(b):
                    w = L[u, j, :, ip]
                    qb = (w[:, None] * qt[u, :, j]).sum(axis=0)
                    if mutation != "unnormalised_query":
                        qb = qb / w.sum()
                    R[u, ip, j] = sm(s * (kt[u, ip] @ qb))
        Ln = np.empty_like(L)
        for u in range(U):
            for j in range(b):
                z = np.empty((mt, mt))
                for i in range(mt):
                    for ip in range(mt):
                        r = R[u, ip, j] if mutation != "transposed_r" else R[u, ip, :, j]
                        kb = r @ kt[u, ip] if mutation != "raw_keys" else kt[u, ip, j]
                        ent = -(r * np.log(r)).sum()
                        if mutation == "no_entropy":
                            ent = 0.0
                        if mutation == "entropy_sign":
                            ent = -ent
                        z[i, ip] = s * (qt[u, i, j] @ kb) + ent
                Ln[u, j] = sm(z)
        L = Ln
    return L, R


def _pins_pass(factors) -> bool:
    ok = True
    q, k, v = _sep()
    for align in ("frame", "row"):
        b = oracle.block_size(GRID, align)
        for steps in (1, 2):
            L, R = factors(q, k, b, None, steps)
            o = mr.factors_matrix(L, R) @ v
            ok &= np.allclose(o, oracle.dense_attention(q, k, v), atol=1e-10)
    q, k, b, tau = _kkt_data()
    L1, R1 = factors(q, k, b, tau, 1)
    L2, R2 = factors(q, k, b, tau, 2)
    ok &= _kkt_gap_l(L1, R1, q, k) < KKT_TOL
    ok &= _kkt_gap_r(L1, R2, q, k) < KKT_TOL
    ok &= _kkt_gap_l(L2, R2, q, k) < KKT_TOL
    return bool(ok)


def test_unmutated_copy_passes_pins():
    assert _pins_pass(lambda q, k, b, tau, steps: _mutant_factors(q, k, b, tau, steps, None))


def test_oracle_factors_pass_pins():
    assert _pins_pass(lambda q, k, b, tau, steps: mr.refine_factors(q, k, b, tau, steps=steps))


@pytest.mark.parametrize("mutation", ["no_entropy", "entropy_sign", "raw_keys", "transposed_r",
                                      "unnormalised_query"])
def test_pins_catch_planted_mistakes(mutation):
    assert not _pins_pass(lambda q, k, b, tau, steps: _mutant_factors(q, k, b, tau, steps, mutation))
