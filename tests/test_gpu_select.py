"""GPU parity of tier assignment: map and order must be bit-exact with the
oracle's when both are fed the same fp32 scores (ties, zeros, sinks, 2-tier,
ragged and maximum request sizes)."""

import numpy as np
import pytest
import torch

from oracle import assign as OA
from oracle import plan as OP
import serving_sk_score_amd as sk
from tests.gpu_helpers import Guarded, say, tied_scores, to_dev, u32

pytestmark = pytest.mark.gpu


def _run(n, S, b, three, scores):
    say("assign", dict(n=n, S=S, b=b, three=three))
    shape = sk.Shape(1, 4, 2, 64)
    pol = sk.Policy(n, S, three, b)
    pl = sk.plan_make(shape, pol)
    opl = OP.make_plan(1, 4, 2, 64, n, S, b, three)
    _, _, amap, order = OA.assign(scores, opl.n16, opl.n8, opl.n4, opl.sinks)
    mg = Guarded(4 * n)
    og = Guarded(4 * n)
    sd = to_dev(scores.astype(np.float32))
    sk.assign_tiers(pol, pl, sd, mg.as_(torch.int32, (n,)), og.as_(torch.int32, (n,)))
    torch.cuda.synchronize()
    mg.check()
    og.check()
    gm = u32(mg.as_(torch.int32, (n,)))
    go = u32(og.as_(torch.int32, (n,)))
    bad = np.nonzero(gm != amap)[0]
    assert bad.size == 0, f"{bad.size} map entries differ, first {bad[:5]}"
    assert np.array_equal(go, order)


@pytest.mark.parametrize("n,S,b,three", [
    (256, 4, 0.5, 1), (1000, 4, 0.3, 1), (1000, 0, 0.3, 1), (777, 4, 0.6, 0),
    (4097, 4, 0.7, 1), (1, 0, 1.0, 1), (2, 1, 0.75, 1), (5, 4, 1.0, 1), (1023, 4, 0.45, 1),
    (1025, 32, 0.35, 1), (8192, 4, 0.5, 1), (32768, 4, 0.6, 0), (32768, 4, 0.3, 1),
    (65536, 4, 0.7, 1), (65536, 4, 0.3, 1), (100003, 4, 0.55, 1),
])
def test_assign_random_with_ties(n, S, b, three):
    _run(n, S, b, three, tied_scores(n + 3, n))


def test_assign_all_equal_and_negative_zero():
    n = 3000
    _run(n, 4, 0.4, 1, np.full(n, 7.25, dtype=np.float32))
    s = np.zeros(n, dtype=np.float32)
    s[::3] = -0.0
    _run(n, 0, 0.6, 1, s)


def test_assign_wide_dynamic_range():
    rng = np.random.default_rng(4)
    n = 20000
    s = (np.exp(rng.uniform(-80, 80, n))).astype(np.float32)
    s[rng.integers(0, n, 500)] = np.float32(1e-45)      # subnormal scores
    _run(n, 4, 0.3, 1, s)


def test_assign_deterministic():
    n = 50000
    s = tied_scores(9, n)
    shape = sk.Shape(1, 4, 2, 64)
    pol = sk.Policy(n, 4, 1, 0.35)
    pl = sk.plan_make(shape, pol)
    sd = to_dev(s)
    outs = []
    for _ in range(2):
        m = torch.empty(n, dtype=torch.int32, device="cuda")
        o = torch.empty(n, dtype=torch.int32, device="cuda")
        sk.assign_tiers(pol, pl, sd, m, o)
        outs.append((m, o))
    torch.cuda.synchronize()
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])
