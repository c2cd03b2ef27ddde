"""Pins for the fp64 oracle: what the pages and the mathematics fix.

Each test checks the oracle against something other than itself: exact
hand-derived values, closed forms, special cases that reduce to a library
routine (torch's scaled_dot_product_attention in float64), invariants, and
brute force on tiny inputs. A final group plants plausible mistakes in a
copy of the oracle's arithmetic and shows that the pins catch each one.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import datagen
import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_examples.json")


def _num(s):
    if s.startswith("ln"):
        return math.log(int(s[2:]))
    return float(Fraction(s))


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


# ---------------------------------------------------------------- golden
@pytest.mark.parametrize("ex", json.load(open(GOLDEN))["examples"], ids=lambda e: e["name"])
def test_hand_examples(ex):
    T, H, W = ex["grid"]
    N = T * H * W
    k = np.array([_num(x) for x in ex["k"]])[:, None]
    v = np.array([_num(x) for x in ex["v"]])[:, None]
    q = np.ones((N, 1))
    want = np.array([float(Fraction(x)) for x in ex["o"]])
    tau = ex["tile_tokens"] or None
    for fn in (oracle.monarch_forward, oracle.monarch_bruteforce):
        got = fn(q, k, v, ex["b"], tau, 1.0)[:, 0]
        np.testing.assert_allclose(got, want, rtol=0, atol=1e-13)
    M = oracle.monarch_matrix(q, k, ex["b"], tau, 1.0)
    np.testing.assert_allclose((M @ v)[:, 0], want, rtol=0, atol=1e-13)


# ---------------------------------------------------------------- V1, V2
SMALL = [  # (grid, b, tau)
    ((4, 2, 3), 6, None),    # frame-aligned, m = 4
    ((4, 2, 3), 3, None),    # row-aligned, m = 8
    ((4, 2, 3), 6, 12),      # tiled: two tiles of 2 frames
    ((4, 2, 3), 24, None),   # dense
    ((4, 2, 3), 1, None),    # token: b = 1
    ((2, 3, 4), 12, 12),     # tau = b: block-diagonal
]


@pytest.mark.parametrize("grid,b,tau", SMALL)
def test_matrix_is_row_stochastic(grid, b, tau):
    N = int(np.prod(grid))
    q, k = _rand((N, 5), 1), _rand((N, 5), 2)
    M = oracle.monarch_matrix(q, k, b, tau)
    assert (M >= 0).all()
    np.testing.assert_allclose(M.sum(axis=1), 1.0, atol=1e-14)
    # nothing crosses a tile
    t = tau or N
    tile = np.arange(N) // t
    assert np.all(M[tile[:, None] != tile[None, :]] == 0)


@pytest.mark.parametrize("grid,b,tau", SMALL)
def test_factored_equals_matrix_equals_bruteforce(grid, b, tau):
    N = int(np.prod(grid))
    q, k, v = _rand((N, 3), 3), _rand((N, 3), 4), _rand((N, 3), 5)
    f = oracle.monarch_forward(q, k, v, b, tau)
    M = oracle.monarch_matrix(q, k, b, tau)
    bf = oracle.monarch_bruteforce(q, k, v, b, tau)
    np.testing.assert_allclose(f, M @ v, atol=1e-13)
    np.testing.assert_allclose(f, bf, atol=1e-13)


def test_every_in_tile_entry_nonzero():
    # "sparsity" is a FLOP saving: the Monarch matrix is dense inside a tile
    q, k = _rand((24, 4), 6), _rand((24, 4), 7)
    M = oracle.monarch_matrix(q, k, 6, None)
    assert (M > 0).all()


# ---------------------------------------------------------------- V3, V4
def _sdpa(q, k, v, mask=None, scale=None):
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a))[None]
    return torch.nn.functional.scaled_dot_product_attention(
        t(q), t(k), t(v), attn_mask=None if mask is None else torch.from_numpy(mask)[None],
        scale=scale)[0].numpy()


@pytest.mark.parametrize("b", [60, 1])
def test_dense_special_cases_match_library(b):
    N, d = 60, 8
    q, k, v = _rand((N, d), 8), _rand((N, d), 9), _rand((N, d), 10)
    got = oracle.monarch_forward(q, k, v, b)
    np.testing.assert_allclose(got, _sdpa(q, k, v), atol=1e-13)
    np.testing.assert_allclose(oracle.dense_attention(q, k, v), _sdpa(q, k, v), atol=1e-13)


def test_tile_equal_block_is_block_diagonal_attention():
    N, d, b = 60, 8, 12
    q, k, v = _rand((N, d), 11), _rand((N, d), 12), _rand((N, d), 13)
    blk = np.arange(N) // b
    mask = blk[:, None] == blk[None, :]
    got = oracle.monarch_forward(q, k, v, b, b)
    np.testing.assert_allclose(got, _sdpa(q, k, v, mask), atol=1e-13)
    np.testing.assert_allclose(oracle.dense_attention(q, k, v, key_tile=b), got, atol=1e-13)


def test_scale_override_and_default():
    N, d = 24, 16
    q, k, v = _rand((N, d), 14), _rand((N, d), 15), _rand((N, d), 16)
    np.testing.assert_allclose(oracle.monarch_forward(q, k, v, N, None, 0.3),
                               _sdpa(q, k, v, scale=0.3), atol=1e-13)
    np.testing.assert_allclose(oracle.monarch_forward(q, k, v, N),
                               _sdpa(q, k, v, scale=1 / 4.0), atol=1e-13)


# ---------------------------------------------------------------- V5, V6
GRID = (3, 4, 5)


def _sep(d=12, seed=17):
    q, k, v = datagen.separable_qkv(1, 1, GRID, d, seed, dtype=torch.float64)
    return q[0, 0].numpy(), k[0, 0].numpy(), v[0, 0].numpy()


@pytest.mark.parametrize("align", ["frame", "row"])
def test_separable_exact_when_aligned(align):
    q, k, v = _sep()
    b = oracle.block_size(GRID, align)
    got = oracle.monarch_forward(q, k, v, b)
    np.testing.assert_allclose(got, oracle.dense_attention(q, k, v), atol=1e-12)


def test_separable_tiled_equals_tile_masked_dense():
    q, k, v = _sep()
    T, H, W = GRID
    # tiles of one frame each with row blocks: tau = H*W, b = W
    got = oracle.monarch_forward(q, k, v, W, H * W)
    np.testing.assert_allclose(got, oracle.dense_attention(q, k, v, key_tile=H * W), atol=1e-12)


def test_misaligned_split_collapses():
    q, k, v = _sep()
    T, H, W = GRID
    dense = oracle.dense_attention(q, k, v)
    err = np.abs(oracle.monarch_forward(q, k, v, 2 * W) - dense).max()  # b = 2W cuts the h axis
    assert err > 0.05, err


def test_separable_generator_logits_decompose():
    # logit(n, n') depends on (t,t'), (h,h'), (w,w') additively
    q, k, _ = _sep()
    T, H, W = GRID
    G = (q @ k.T).reshape(T, H, W, T, H, W)
    # second differences across axes vanish for an additive form
    mixed = G[1, 0, 0, 1, 0, 0] - G[1, 0, 0, 0, 0, 0] - G[0, 0, 0, 1, 0, 0] + G[0, 0, 0, 0, 0, 0]
    assert abs(mixed) > 1e-3  # t-t' interaction exists
    x = G[:, :, :, 0, 0, 0]
    assert np.allclose(x[1, 1, 0] - x[1, 0, 0] - x[0, 1, 0] + x[0, 0, 0], 0, atol=1e-12)


# ---------------------------------------------------------------- V7, V8
@pytest.mark.parametrize("which", ["q", "k"])
def test_zero_logits_give_tile_mean(which):
    T, H, W = 4, 2, 3
    N, d = 24, 5
    q, k, v = _rand((N, d), 18), _rand((N, d), 19), _rand((N, d), 20)
    if which == "q":
        q[:] = 0
    else:
        k[:] = 0
    for b, tau in [(6, None), (3, None), (6, 12)]:
        t = tau or N
        want = np.repeat(v.reshape(N // t, t, d).mean(axis=1), t, axis=0)
        np.testing.assert_allclose(oracle.monarch_forward(q, k, v, b, tau), want, atol=1e-14)


def test_constant_values_pass_through():
    N, d = 24, 5
    q, k = _rand((N, d), 21), _rand((N, d), 22)
    v = np.tile(_rand((1, d), 23), (N, 1))
    np.testing.assert_allclose(oracle.monarch_forward(q, k, v, 6), v, atol=1e-14)


# ---------------------------------------------------------------- V9
def test_inblock_permutation_equivariance():
    N, d, b = 24, 4, 6
    q, k, v = _rand((N, d), 24), _rand((N, d), 25), _rand((N, d), 26)
    sigma = np.random.default_rng(0).permutation(b)
    perm = (np.arange(N) // b) * b + sigma[np.arange(N) % b]
    o = oracle.monarch_forward(q, k, v, b)
    op = oracle.monarch_forward(q[perm], k[perm], v[perm], b)
    np.testing.assert_allclose(op, o[perm], atol=1e-13)


def test_block_and_tile_permutation_equivariance():
    N, d, b, tau = 24, 4, 3, 12
    q, k, v = _rand((N, d), 27), _rand((N, d), 28), _rand((N, d), 29)
    o = oracle.monarch_forward(q, k, v, b, tau)
    rng = np.random.default_rng(1)
    pi = rng.permutation(tau // b)  # blocks within each tile
    n = np.arange(N)
    perm = (n // tau) * tau + pi[(n % tau) // b] * b + n % b
    np.testing.assert_allclose(oracle.monarch_forward(q[perm], k[perm], v[perm], b, tau), o[perm], atol=1e-13)
    tp = (1 - n // tau) * tau + n % tau  # swap the two tiles
    np.testing.assert_allclose(oracle.monarch_forward(q[tp], k[tp], v[tp], b, tau), o[tp], atol=1e-13)


def test_different_permutation_per_block_is_not_equivariant():
    N, d, b = 24, 4, 6
    q, k, v = _rand((N, d), 30), _rand((N, d), 31), _rand((N, d), 32)
    rng = np.random.default_rng(2)
    perm = np.concatenate([i * b + rng.permutation(b) for i in range(N // b)])
    o = oracle.monarch_forward(q, k, v, b)
    op = oracle.monarch_forward(q[perm], k[perm], v[perm], b)
    assert np.abs(op - o[perm]).max() > 0.05


# ---------------------------------------------------------------- V10 and plan arithmetic
def test_flop_count_matches_the_pages_sparsity():
    # frame-aligned 21x30x52 grid: (b + m)/N of the dense QK^T/PV work, which
    # the pages put at 5% ("95% sparsity")
    N, b, m = 21 * 30 * 52, 1560, 21
    dense = 4 * 12 * N * 128 * N
    f = oracle.flop_count(1, 12, N, 128, b, m)
    assert f == 48 * 32760 * 128 * 1581 == 318_219_632_640
    assert abs(1 - f / dense - 0.9517) < 1e-3
    assert oracle.flop_count(1, 1, 8, 1, 2, 2) == 4 * 8 * (2 + 2)


def test_block_sizes_and_plan_checks():
    g = (21, 30, 52)
    assert oracle.block_size(g, "frame") == 1560
    assert oracle.block_size(g, "row") == 52
    assert oracle.block_size(g, "dense") == 32760
    assert oracle.block_size(g, "token") == 1
    oracle.check_plan(32760, 1560, 4680)
    for bad in [(32760, 1000, 32760), (32760, 1560, 3000), (32760, 1560, 1560 * 4)]:
        with pytest.raises(ValueError):
            oracle.check_plan(*bad)


def test_sampled_groups_match_full():
    N, d, b, tau = 24, 4, 3, 12
    q, k, v = _rand((2, N, d), 33), _rand((2, N, d), 34), _rand((2, N, d), 35)
    full = oracle.monarch_forward(q, k, v, b, tau)
    res = oracle.monarch_forward_groups(q, k, v, b, tau, None, [0, 1], [(0, 0), (1, 2)])
    for (h, u, j), (idx, rows) in res.items():
        np.testing.assert_allclose(rows, full[h, idx], atol=1e-13)


# ---------------------------------------------------------------- input generator
def test_positional_code():
    d = 128
    assert datagen.axis_channels(d) == (44, 42, 42)
    pe = datagen.positional_code(3, 4, 5, d)
    assert pe.shape == (60, d)
    # sin^2 + cos^2 = 1 per frequency: every row has squared norm d/2
    np.testing.assert_allclose((pe ** 2).sum(axis=1), d / 2, atol=1e-12)
    # token 0 is (0,0,0): sines 0, cosines 1
    assert np.allclose(pe[0, :22], 0) and np.allclose(pe[0, 22:44], 1)
    # the w part of token n depends only on n % W
    assert np.allclose(pe[7, 86:], pe[2, 86:])


def test_generator_is_seeded_and_prefix_stable():
    a = datagen.qkv(1, 3, (2, 3, 4), 64, (5, 6, 7))
    b = datagen.qkv(1, 1, (2, 3, 4), 64, (5, 6, 7))
    assert all(x.dtype == torch.bfloat16 for x in a)
    assert torch.equal(a[0][:, :1], b[0])


# ---------------------------------------------------------------- planted mistakes
def _mutant_forward(q, k, v, b, tau, mutation):
    """A copy of the factored arithmetic with one planted mistake."""
    N, d = q.shape
    s = 1 / math.sqrt(d) if mutation != "no_scale" else 1.0
    nb = N // b
    U, mt = N // tau, tau // b
    sm = oracle.softmax_rows

    def st1(qq, kk, vv):
        qb, kb, vb = (x.reshape(nb, b, d) for x in (qq, kk, vv))
        return np.matmul(sm(s * qb @ kb.transpose(0, 2, 1)), vb).reshape(N, d)

    def st2(qq, kk, yy):
        g = lambda x: x.reshape(U, mt, b, d).transpose(0, 2, 1, 3)
        if mutation == "contiguous_groups":
            g = lambda x: x.reshape(U, b, mt, d)
        qg, kg, yg = g(qq), g(kk), g(yy)
        p = sm(s * qg @ kg.transpose(0, 1, 3, 2))
        if mutation == "transposed_p2":
            p = p.transpose(0, 1, 3, 2)
        o = p @ yg
        if mutation == "contiguous_groups":
            return o.reshape(N, d)
        return o.transpose(0, 2, 1, 3).reshape(N, d)

    if mutation == "stages_swapped":
        return st1(q, k, st2(q, k, v))
    if mutation == "stage2_reads_v":
        return st2(q, k, v)
    return st2(q, k, st1(q, k, v))


def _pins_pass(fwd) -> bool:
    """Run the separable, golden and brute-force pins against ``fwd``."""
    ok = True
    q, k, v = _sep()
    for align in ("frame", "row"):
        b = oracle.block_size(GRID, align)
        ok &= np.allclose(fwd(q, k, v, b, 60), oracle.dense_attention(q, k, v), atol=1e-10)
    N = 24
    qq, kk, vv = _rand((N, 3), 40), _rand((N, 3), 41), _rand((N, 3), 42)
    ok &= np.allclose(fwd(qq, kk, vv, 6, 24), oracle.monarch_bruteforce(qq, kk, vv, 6), atol=1e-12)
    for ex in json.load(open(GOLDEN))["examples"]:
        T, H, W = ex["grid"]
        n = T * H * W
        kk = np.array([_num(x) for x in ex["k"]])[:, None]
        vv = np.array([_num(x) for x in ex["v"]])[:, None]
        want = np.array([float(Fraction(x)) for x in ex["o"]])
        got = fwd(np.ones((n, 1)), kk, vv, ex["b"], ex["tile_tokens"] or n)[:, 0]
        ok &= np.allclose(got, want, atol=1e-12)
    return bool(ok)


def test_unmutated_copy_passes_pins():
    assert _pins_pass(lambda q, k, v, b, tau: _mutant_forward(q, k, v, b, tau, None))


@pytest.mark.parametrize("mutation", ["no_scale", "contiguous_groups", "transposed_p2",
                                      "stages_swapped", "stage2_reads_v"])
def test_pins_catch_planted_mistakes(mutation):
    assert not _pins_pass(lambda q, k, v, b, tau: _mutant_forward(q, k, v, b, tau, mutation))
