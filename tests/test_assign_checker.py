"""The property checker that the tier-selection test at the token limit uses
in place of the oracle's sort: it accepts the oracle's assignment and
rejects a planted mistake of each kind it is there to catch (a ranking
error with an otherwise consistent map and order, slots out of token order,
a sink outside fp16, wrong tier counts).  CPU only; the mistakes are planted
in the oracle's output."""

import numpy as np
import pytest

from oracle import assign as OA
from oracle import plan as OP
from tests.test_gpu_select import _check_assignment

N, S = 200_003, 4


def _fails(scores, counts, gm, go):
    with pytest.raises(AssertionError):
        _check_assignment(scores, S, counts, gm, go, chunk=1 << 14, threads=4)


@pytest.mark.parametrize("b,three,overflow", [(0.45, 1, 0), (0.7, 1, 0), (0.3, 0, 1)])
def test_checker_accepts_oracle_and_catches_planted_mistakes(b, three, overflow):
    rng = np.random.default_rng(11)
    # about 12 tokens per distinct value, so every tier boundary is a tie
    scores = (rng.integers(0, N // 12, N) / 1024.0).astype(np.float32)
    pl = OP.make_plan(1, 1, 1, 64, N, S, b, three, overflow=overflow)
    counts = np.array([pl.n16, pl.n8, pl.n4, N - pl.n16 - pl.n8 - pl.n4])
    _, _, amap, order = OA.assign(scores, pl.n16, pl.n8, pl.n4, pl.sinks)
    _check_assignment(scores, S, counts, amap, order, chunk=1 << 14, threads=4)

    tier = amap >> 30
    # ranking: the oracle's assignment of scores in which the last-ranked
    # token of a tier and the first-ranked of the next trade places
    hi = 0 if counts[0] > S else 1
    lo = hi + 1 if counts[hi + 1] else hi + 2
    th = np.nonzero(tier == hi)[0]
    th = th[th >= S]
    tl = np.nonzero(tier == lo)[0]
    a = th[np.lexsort((-th, scores[th]))[0]]
    c = tl[np.lexsort((tl, -scores[tl]))[0]]
    s2 = scores.copy()
    s2[a], s2[c] = scores[c] * np.float32(0.5), scores[a] * np.float32(2) + np.float32(1)
    _, _, m2, o2 = OA.assign(s2, pl.n16, pl.n8, pl.n4, pl.sinks)
    _fails(scores, counts, m2, o2)

    # two tokens of one tier with their slots (and order entries) exchanged
    j = np.nonzero(tier == 1)[0][:2]
    gm, go = amap.copy(), order.copy()
    gm[j[0]], gm[j[1]] = gm[j[1]], gm[j[0]]
    p, q = (np.nonzero(order == x)[0][0] for x in j)
    go[p], go[q] = go[q], go[p]
    _fails(scores, counts, gm, go)

    # a sink sent at int8, and counts that disagree with the plan
    gm = amap.copy()
    gm[0] = 1 << 30
    _fails(scores, counts, gm, order)
    _fails(scores, counts + np.array([1, -1, 0, 0]), amap, order)
