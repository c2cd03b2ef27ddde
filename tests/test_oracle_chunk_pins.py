"""Pins for the oracle of one frame-causal chunk (no GPU).

The chunk reading: stage 1 unchanged; each stage-2 group keeps its rows of
frames before t1 as keys/values and the chunk's rows as queries. Pinned by:
the whole video as one chunk is the ordinary forward; explicit loops over
tokens (the factor formulas written out) on tiny inputs; frames from t1 on
have no influence; a first frame alone reduces to its stage-1 output (a
softmax over a single key is 1).
"""
import numpy as np
import pytest

import oracle

RNG = np.random.default_rng(77)


def rand(*shape):
    return RNG.standard_normal(shape)


@pytest.mark.parametrize("grid,align", [((5, 3, 4), "frame"), ((5, 3, 4), "row"), ((4, 2, 3), "token")])
def test_whole_video_chunk_is_the_forward(grid, align):
    T, H, W = grid
    N, d = T * H * W, 6
    b = oracle.block_size(grid, align)
    q, k, v = rand(2, N, d), rand(2, N, d), rand(2, N, d)
    got = oracle.monarch_chunk_forward(q, k, v, b, H * W, 0, T)
    np.testing.assert_allclose(got, oracle.monarch_forward(q, k, v, b), rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("grid,align,t0,t1", [((4, 2, 3), "frame", 1, 3), ((4, 2, 3), "frame", 3, 4),
                                              ((4, 2, 3), "row", 0, 2), ((4, 2, 3), "row", 2, 4),
                                              ((3, 2, 2), "token", 1, 2)])
def test_chunk_matches_token_loops(grid, align, t0, t1):
    T, H, W = grid
    N, d = T * H * W, 3
    b = oracle.block_size(grid, align)
    q, k, v = rand(N, d), rand(N, d), rand(N, d)
    got = oracle.monarch_chunk_forward(q, k, v, b, H * W, t0, t1)
    want = oracle.monarch_chunk_bruteforce(q, k, v, b, H * W, t0, t1)
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("align", ["frame", "row"])
def test_future_frames_have_no_influence(align):
    grid = (6, 3, 4)
    T, H, W = grid
    N, d = T * H * W, 5
    b = oracle.block_size(grid, align)
    q, k, v = rand(N, d), rand(N, d), rand(N, d)
    t0, t1 = 2, 4
    a = oracle.monarch_chunk_forward(q, k, v, b, H * W, t0, t1)
    q2, k2, v2 = q.copy(), k.copy(), v.copy()
    for x in (q2, k2, v2):
        x[t1 * H * W:] = rand(N - t1 * H * W, d) * 10
    np.testing.assert_array_equal(a, oracle.monarch_chunk_forward(q2, k2, v2, b, H * W, t0, t1))
    # ... while the queries of the chunk and the keys of earlier frames do matter
    k2 = k.copy()
    k2[:H * W] += 1.0
    assert not np.allclose(a, oracle.monarch_chunk_forward(q, k2, v, b, H * W, t0, t1))


def test_first_frame_alone_is_its_stage1_output():
    grid = (4, 3, 5)
    T, H, W = grid
    N, d = T * H * W, 8
    q, k, v = rand(N, d), rand(N, d), rand(N, d)
    got = oracle.monarch_chunk_forward(q, k, v, H * W, H * W, 0, 1)
    y = oracle.stage1(q[:H * W], k[:H * W], v[:H * W], H * W, d ** -0.5)
    np.testing.assert_allclose(got, y, rtol=1e-12, atol=1e-12)


def test_planted_mistake_dropping_the_current_chunk_keys_fails():
    grid = (4, 2, 3)
    T, H, W = grid
    N, d = T * H * W, 3
    q, k, v = rand(N, d), rand(N, d), rand(N, d)
    good = oracle.monarch_chunk_forward(q, k, v, H * W, H * W, 2, 3)
    # a reading where a chunk sees only earlier chunks plus itself frame by frame
    # (frame-causal inside the chunk) differs as soon as the chunk has 2+ frames
    bad = np.concatenate([oracle.monarch_chunk_forward(q, k, v, H * W, H * W, t, t + 1) for t in (2,)])
    np.testing.assert_allclose(good, bad, atol=1e-12)  # one-frame chunk: the two readings agree
    good2 = oracle.monarch_chunk_forward(q, k, v, H * W, H * W, 1, 3)
    bad2 = np.concatenate([oracle.monarch_chunk_forward(q, k, v, H * W, H * W, t, t + 1) for t in (1, 2)])
    assert not np.allclose(good2, bad2)
