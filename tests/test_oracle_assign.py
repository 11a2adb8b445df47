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


# ------------------------------------------------- drops and variants --

def test_dropped_tokens_are_the_lowest_ranked():
    rng = np.random.default_rng(12)
    for trial in range(30):
        n = int(rng.integers(1, 300))
        S = int(rng.integers(0, min(n, 6) + 1))
        sc = (rng.integers(0, 20, size=n) * 0.25).astype(np.float32)   # many ties
        n16 = S + int(rng.integers(0, n - S + 1))
        n8 = int(rng.integers(0, n - n16 + 1))
        n4 = int(rng.integers(0, n - n16 - n8 + 1))
        tier, slot, amap, order = A.assign(sc, n16, n8, n4, S)
        # brute force with Python's sort: rank by (score desc, index asc)
        ranked = sorted(range(S, n), key=lambda j: (-float(sc[j]), j))
        want = [0] * S + [None] * (n - S)
        cuts = [n16 - S, n16 - S + n8, n16 - S + n8 + n4]
        for r, j in enumerate(ranked):
            want[j] = 0 if r < cuts[0] else 1 if r < cuts[1] else 2 if r < cuts[2] else 3
        assert list(tier) == want, trial
        assert np.sum(tier == 3) == n - n16 - n8 - n4
        # dropped tokens take slots in token order and close the order list
        drop = np.nonzero(tier == 3)[0]
        assert list(slot[drop]) == list(range(len(drop)))
        assert list(order[n - len(drop):]) == list(drop)
        assert np.all((amap >> 30)[drop] == 3)


def test_balanced_power_of_two_is_strided():
    keys = A.balanced_keys(64 + 3, 3)                 # 3 sinks, R = 64
    assert np.all(keys[:3] == 0)
    tier, _, _, _ = A.assign(keys, 3 + 16, 16, 32, 3)
    r = np.arange(64)
    assert np.array_equal(np.nonzero(tier[3:] == 0)[0], r[r % 4 == 0])
    assert np.array_equal(np.nonzero(tier[3:] <= 1)[0], r[r % 2 == 0])


def test_balanced_spreads_every_tier_boundary():
    for R in (5, 100, 1000, 1025):
        keys = A.balanced_keys(R, 0)
        assert len(np.unique(keys)) == R                  # a strict ranking, no ties
        b = int(np.ceil(np.log2(R)))
        order = sorted(range(R), key=lambda j: -float(keys[j]))
        w = np.arange(1, R + 1)
        for k in range(1, R, max(1, R // 50)):
            sel = np.zeros(R, dtype=bool)
            sel[order[:k]] = True
            dev = np.max(np.abs(np.cumsum(sel) - w * k / R))
            assert dev <= b / 2, (R, k, dev)              # position-greedy would be ~k(R-k)/R
