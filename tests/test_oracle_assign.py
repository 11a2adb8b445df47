"""Pins of the oracle's tier assignment.

What fixes the expected values: brute force over every assignment with the
plan's tier counts (the SpectrumKV paper's §2.3 Proposition 1: the sorted
assignment minimises the importance-weighted error for any increasing
per-tier error), sinks pinned to fp16 (§7.4.1), and 2-tier mode never
producing int4 (§4.5).
"""

import itertools

import numpy as np
import pytest

from oracle import assign as A
from oracle import plan as P


def _brute(score, n16, n8, n4, sinks, delta):
    n = len(score)
    best = None
    tiers0 = [0] * sinks
    pool = [0] * (n16 - sinks) + [1] * n8 + [2] * n4
    for perm in set(itertools.permutations(pool)):
        t = tiers0 + list(perm)
        err = A.weighted_error(score, t, delta)
        key = (round(err, 9), t)          # among minimisers prefer lower tiers at lower indices
        if best is None or key < best:
            best = key
    return best[1]


def test_brute_force_proposition_1():
    rnd = np.random.default_rng(0)
    cases = 0
    for n in range(1, 8):
        for sinks in (0, 1, 2):
            if sinks > n:
                continue
            for _ in range(6):
                score = rnd.integers(0, 4, size=n).astype(np.float32)   # deliberate ties
                R = n - sinks
                a = int(rnd.integers(0, R + 1))
                c = int(rnd.integers(0, R - a + 1))
                n16, n8, n4 = sinks + a, c, R - a - c
                tier, slot, amap, order = A.assign(score, n16, n8, n4, sinks)
                for delta in ((0, 1, 3), (0, 2, 3)):
                    want = _brute(score, n16, n8, n4, sinks, delta)
                    assert list(tier) == want, (score, n16, n8, n4, sinks)
                cases += 1
    assert cases > 100


def test_sinks_slots_order_invariants():
    rnd = np.random.default_rng(1)
    for n, S, b, three in [(256, 4, 0.5, 1), (1000, 4, 0.3, 1), (513, 0, 0.7, 1), (777, 4, 0.6, 0), (64, 64, 1.0, 1)]:
        N16, N8, N4, s = P.tier_counts(n, S, b, three)
        score = rnd.random(n).astype(np.float32)
        score[5:20] = score[4]                                  # ties
        tier, slot, amap, order = A.assign(score, N16, N8, N4, s)
        assert np.all(tier[:s] == P.FP16)
        assert np.array_equal(slot[:s], np.arange(s))
        assert [int((tier == t).sum()) for t in (0, 1, 2)] == [N16, N8, N4]
        if not three:
            assert not np.any(tier == P.INT4)
        for t in (0, 1, 2):
            members = np.nonzero(tier == t)[0]
            assert np.array_equal(slot[members], np.arange(len(members)))
        assert np.array_equal(amap >> 30, tier) and np.array_equal(amap & ((1 << 30) - 1), slot)
        # order = tokens sorted by (tier, index)
        assert sorted(order.tolist()) == list(range(n))
        key = [(tier[j], j) for j in order]
        assert key == sorted(key)
        # monotone: every non-sink fp16 score >= every int8 score >= every int4 score
        ns = np.arange(n) >= s
        for hi, lo in ((0, 1), (1, 2)):
            a = score[ns & (tier == hi)]
            bb = score[ns & (tier == lo)]
            if len(a) and len(bb):
                assert a.min() >= bb.max()


def test_tie_break_lower_index_first():
    score = np.array([0, 5, 5, 5, 5, 1], dtype=np.float32)
    tier, *_ = A.assign(score, 2, 2, 2, 0)
    assert list(tier) == [2, 0, 0, 1, 1, 2]


def test_negative_zero_is_zero():
    score = np.array([-0.0, 0.0, 0.0], dtype=np.float32)
    tier, *_ = A.assign(score, 1, 1, 1, 0)
    assert list(tier) == [0, 1, 2]


def test_rejects_nonfinite():
    with pytest.raises(AssertionError):
        A.assign(np.array([1.0, np.nan], dtype=np.float32), 1, 1, 0, 0)
