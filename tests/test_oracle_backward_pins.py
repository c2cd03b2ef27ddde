"""Pins for the fp64 backward oracle (no GPU).

The backward oracle is the chain rule written out by hand; these tests tie
it to things it does not share code with:
  * central finite differences of the forward oracle (no gradient formula);
  * torch autograd (fp64) of a forward written here from the spec with torch
    ops, which differentiates the definition mechanically;
  * the dense special case (b = N) against torch's own scaled-dot-product
    attention, differentiated by autograd;
  * closed forms and invariants: dV column sums equal G column sums (every
    row of the Monarch matrix sums to 1); constant V rows give dQ = dK = 0;
    per tile, the keys' gradient sums to zero (softmax is invariant under a
    shift of all logits of a row).
Planted mistakes (a dropped softmax-Jacobian term, a transposed product, a
missing stage) must fail the pins.
"""
import numpy as np
import pytest
import torch

import datagen
import oracle

RNG = np.random.default_rng(1234)


def rand(*shape):
    return RNG.standard_normal(shape)


def loss(q, k, v, g, b, tile=None, scale=None):
    return float(np.sum(g * oracle.monarch_forward(q, k, v, b, tile, scale)))


CASES = [  # (grid, d, b, tile)
    ((2, 2, 3), 4, 6, None),      # frame: 2 blocks of 6, groups of 2
    ((2, 3, 2), 3, 2, None),      # row: 6 blocks of 2, groups of 6
    ((4, 1, 2), 3, 2, 4),         # tiled: 2 tiles of 2 blocks
    ((3, 1, 2), 2, 6, None),      # dense (b = N)
    ((3, 1, 2), 2, 1, None),      # token (b = 1): stage 2 alone
]


@pytest.mark.parametrize("grid,d,b,tile", CASES)
def test_backward_matches_central_differences(grid, d, b, tile):
    N = grid[0] * grid[1] * grid[2]
    q, k, v, g = (rand(N, d) for _ in range(4))
    dq, dk, dv = oracle.monarch_backward(q, k, v, g, b, tile)
    h = 1e-6
    for x, dx in ((q, dq), (k, dk), (v, dv)):
        num = np.empty_like(x)
        for idx in np.ndindex(*x.shape):
            old = x[idx]
            x[idx] = old + h
            lp = loss(q, k, v, g, b, tile)
            x[idx] = old - h
            lm = loss(q, k, v, g, b, tile)
            x[idx] = old
            num[idx] = (lp - lm) / (2 * h)
        np.testing.assert_allclose(dx, num, rtol=1e-6, atol=1e-8)


def torch_monarch(q, k, v, b, tau, s):
    """The forward spec in torch ops (fp64), for autograd: blocks, then groups."""
    N, d = q.shape
    blk = lambda x: x.reshape(N // b, b, d)
    p1 = torch.softmax(s * blk(q) @ blk(k).transpose(1, 2), dim=-1)
    y = (p1 @ blk(v)).reshape(N, d)
    U, mt = N // tau, tau // b
    grp = lambda x: x.reshape(U, mt, b, d).permute(0, 2, 1, 3)
    p2 = torch.softmax(s * grp(q) @ grp(k).transpose(2, 3), dim=-1)
    return (p2 @ grp(y)).permute(0, 2, 1, 3).reshape(N, d)


@pytest.mark.parametrize("grid,align,tile", [((3, 4, 5), "frame", None), ((3, 4, 5), "row", None),
                                             ((6, 2, 5), "frame", 30), ((4, 3, 4), "row", 24)])
def test_backward_matches_torch_autograd(grid, align, tile):
    N, d = grid[0] * grid[1] * grid[2], 8
    b = oracle.block_size(grid, align)
    q, k, v, g = (rand(N, d) for _ in range(4))
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    out = torch_monarch(tq, tk, tv, b, tile or N, d ** -0.5)
    out.backward(torch.tensor(g))
    dq, dk, dv = oracle.monarch_backward(q, k, v, g, b, tile)
    for mine, ref in ((dq, tq.grad), (dk, tk.grad), (dv, tv.grad)):
        np.testing.assert_allclose(mine, ref.numpy(), rtol=1e-10, atol=1e-12)


def test_dense_case_matches_sdpa_autograd():
    N, d = 40, 16
    q, k, v, g = (rand(N, d) for _ in range(4))
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    out = torch.nn.functional.scaled_dot_product_attention(tq[None], tk[None], tv[None])[0]
    out.backward(torch.tensor(g))
    for b in (N, 1):  # one block (stage 2 is the identity) and one token per block
        dq, dk, dv = oracle.monarch_backward(q, k, v, g, b)
        np.testing.assert_allclose(dq, tq.grad.numpy(), rtol=1e-9, atol=1e-11)
        np.testing.assert_allclose(dk, tk.grad.numpy(), rtol=1e-9, atol=1e-11)
        np.testing.assert_allclose(dv, tv.grad.numpy(), rtol=1e-9, atol=1e-11)


@pytest.mark.parametrize("align,tile", [("frame", None), ("row", None), ("frame", 60)])
def test_invariants(align, tile):
    grid, d = (4, 3, 5), 8
    N = 60
    b = oracle.block_size(grid, align)
    q, k, v, g = (rand(N, d) for _ in range(4))
    dq, dk, dv = oracle.monarch_backward(q, k, v, g, b, tile)
    tau = tile or N
    # every row of M sums to 1, so sum_n' dV[n'] = sum_n G[n] (per tile)
    np.testing.assert_allclose(dv.reshape(-1, tau, d).sum(1), g.reshape(-1, tau, d).sum(1), atol=1e-12)
    # shifting every key of a problem by one vector leaves P unchanged: the
    # keys' gradient sums to zero over every block and every group, so per tile
    np.testing.assert_allclose(dk.reshape(-1, tau, d).sum(1), 0, atol=1e-12)
    # constant value rows: O does not depend on Q or K at all
    vc = np.tile(rand(1, d), (N, 1))
    dq0, dk0, dv0 = oracle.monarch_backward(q, k, vc, g, b, tile)
    np.testing.assert_allclose(dq0, 0, atol=1e-12)
    np.testing.assert_allclose(dk0, 0, atol=1e-12)


def test_planted_mistakes_fail_the_pins():
    N, d, b = 12, 4, 6
    q, k, v, g = (rand(N, d) for _ in range(4))
    s = d ** -0.5
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    torch_monarch(tq, tk, tv, b, N, s).backward(torch.tensor(g))
    good = oracle.monarch_backward(q, k, v, g, b)
    assert np.allclose(good[0], tq.grad.numpy(), atol=1e-10)

    def wrong_attention_backward(q_, k_, v_, g_, scale, mistake):
        kt = np.swapaxes(k_, -1, -2)
        p = oracle.softmax_rows(scale * np.matmul(q_, kt))
        o = np.matmul(p, v_)
        dv_ = np.matmul(np.swapaxes(p, -1, -2), g_)
        dp = np.matmul(g_, np.swapaxes(v_, -1, -2))
        delta = 0 if mistake == "no_delta" else np.sum(g_ * o, axis=-1, keepdims=True)
        ds = p * (dp - delta)
        dq_ = scale * (np.matmul(np.swapaxes(ds, -1, -2), k_) if mistake == "transposed" else np.matmul(ds, k_))
        dk_ = scale * np.matmul(np.swapaxes(ds, -1, -2), q_)
        return dq_, dk_, dv_

    import sys
    mb = sys.modules["oracle.monarch_backward"]  # the module (the package re-exports a function of that name)
    orig = mb.attention_backward
    for mistake in ("no_delta", "transposed"):
        mb.attention_backward = lambda *a, m=mistake: wrong_attention_backward(*a, m)
        try:
            bad = mb.monarch_backward(q, k, v, g, b)
        finally:
            mb.attention_backward = orig
        assert not np.allclose(bad[0], tq.grad.numpy(), atol=1e-6), mistake
    # a forgotten stage: stage-2 gradients alone (as if dQ1 were dropped)
    y = oracle.stage1(q, k, v, b, s)
    dq2, _, _ = oracle.stage2_backward(q, k, y, g, b, N, s)
    assert not np.allclose(dq2, tq.grad.numpy(), atol=1e-6)


def test_backward_on_generator_inputs_is_finite():
    q, k, v = datagen.qkv(1, 2, (3, 4, 10), 16, (5, 6, 7), dtype=torch.bfloat16)
    g = datagen.qkv(1, 2, (3, 4, 10), 16, (8, 9, 10), dtype=torch.bfloat16)[0]
    for x in oracle.monarch_backward(q, k, v, g, 40):
        assert np.isfinite(x).all() and x.shape == (1, 2, 120, 16)
