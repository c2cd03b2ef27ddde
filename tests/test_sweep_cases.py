"""Host logic of the alignment / tile sweep, and the sweep's claims on the oracle.

The sweep (structured_attention_video_amd/sweep.py) measures on the GPU what
the MonarchRT pages claim qualitatively (gist.science explainer, Methodology A
and B): aligned blocks keep the separable part of the logits exactly,
misaligned blocks do not. Here the same cases and input families are run
through the fp64 oracle at a small size, so the claims the GPU sweep reports
are pinned on the oracle, not on the kernels.
"""
import math

import numpy as np
import pytest

import datagen
import oracle
from structured_attention_video_amd.sweep import FAMILIES, block_cases, divisors, rel_l2, tile_counts


def test_divisors():
    assert divisors(1) == [1]
    assert divisors(12) == [1, 2, 3, 4, 6, 12]
    assert divisors(32760)[:6] == [1, 2, 3, 4, 5, 6] and len(divisors(32760)) == 96


def test_block_cases_frame_shape():
    cases = block_cases((21, 30, 52))
    assert cases[0] == ("frame", "frame", 0, 1560) and cases[1] == ("row", "row", 0, 52)
    mis = [c for c in cases if c[1] == "custom"]
    assert [c[0] for c in mis] == ["misaligned~frame", "misaligned~row"]
    for _, _, cb, b in mis:
        assert cb == b and 32760 % b == 0 and b % 52 and 52 % b  # divides N, straddles rows
    # nearest in ratio among the straddling divisors
    assert mis[0][3] == 1638 and mis[1][3] == 56


def test_block_cases_small_and_tiles():
    cases = block_cases((4, 6, 10))
    assert [c[3] for c in cases] == [60, 10, 48, 12]
    assert tile_counts(21) == [1, 3, 7, 21] and tile_counts(4) == [1, 2, 4]


def test_rel_l2():
    import torch
    a = torch.tensor([3.0, 4.0])
    assert rel_l2(a, a) == 0.0
    assert math.isclose(rel_l2(torch.tensor([3.0, 5.0]), a), 0.2, rel_tol=1e-6)  # fp32


def oracle_rel_errors(grid, family, d=64, heads=1):
    """rel-L2 of the oracle's Monarch output against its dense output, per block case."""
    make = dict(FAMILIES)[family]
    q, k, v = make(grid, heads, d)
    q, k, v = (x.float() for x in (q, k, v))
    dense = np.stack([oracle.dense_attention(q[0, h], k[0, h], v[0, h]) for h in range(heads)])
    out = {}
    for label, _, _, b in block_cases(grid):
        mon = oracle.monarch_forward(q[0], k[0], v[0], b)
        out[label] = float(np.linalg.norm(mon - dense) / np.linalg.norm(dense))
    return out


def test_oracle_separable_aligned_exact_misaligned_not():
    e = oracle_rel_errors((4, 6, 10), "separable")
    assert e["frame"] < 1e-6 and e["row"] < 1e-6  # exact up to the bf16 inputs' fp64 arithmetic
    assert e["misaligned~frame"] > 0.05 and e["misaligned~row"] > 0.05


def test_oracle_noisy_separable_aligned_beats_misaligned():
    e = oracle_rel_errors((4, 6, 10), "separable+noise0.5")
    assert max(e["frame"], e["row"]) < min(e["misaligned~frame"], e["misaligned~row"])
