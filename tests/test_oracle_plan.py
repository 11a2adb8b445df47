"""Pins of the oracle's budget -> tier-count rule and payload size.

What fixes the expected values:
* the SpectrumKV paper's printed consequences of the §4.4 mapping
  (b=0.3 -> about 80% int4, §6.2; b=0.5 -> every token int8, §6.1 and §7.5;
  b=0.25 -> every token int4, §7.5; the 2-tier policy at b=0.3 can send only
  60% of the tokens at int8, §7.4.3);
* the §2.1 closed form for the fp16 volume;
* brute force over every feasible triple for small n;
* exact rational arithmetic for the budget;
* the Minima-KV page's printed accounting (18.3 KiB/token = 4.58 bits per
  scalar, 3.497x against BF16) for the bits-per-scalar formula.
"""

import itertools
import math
from fractions import Fraction

import numpy as np
import pytest

from oracle import plan as P


@pytest.mark.parametrize("b,expect", [
    (0.3, (0, 200, 800)),      # §6.2: "roughly 80% of tokens in int4"
    (0.5, (0, 1000, 0)),       # §6.1 / §7.5: b=0.5 is all-token int8
    (0.25, (0, 0, 1000)),      # §7.5: uniform int4 corresponds to b=0.25
])
def test_printed_cases_no_sinks(b, expect):
    N16, N8, N4, s = P.tier_counts(1000, 0, b, 1)
    assert (N16, N8, N4) == expect and s == 0


@pytest.mark.parametrize("b", [0.25, 0.3, 0.35, 0.4, 0.45, 0.5])
def test_section_4_4_fractions(b):
    # §4.4: f8 = 4b - 1, f4 = 2 - 4b, f16 = 0 (S = 0, 4bn integral)
    n = 2000
    N16, N8, N4, _ = P.tier_counts(n, 0, b, 1)
    assert N16 == 0
    assert Fraction(N8, n) == Fraction(str(b)) * 4 - 1
    assert Fraction(N4, n) == 2 - 4 * Fraction(str(b))
    # §2.1 costs: the whole budget is used exactly
    assert Fraction(N8, 2) + Fraction(N4, 4) == Fraction(str(b)) * n


def test_two_tier_sixty_percent():
    # §7.4.3: at b=0.3 int8 costs 1/2, so only 60% of the tokens fit at int8;
    # the oracle rejects such a budget instead of dropping tokens.
    n = 1000
    B = P.budget_units(0.3, n)
    assert B // P.UNITS[P.INT8] == 600
    with pytest.raises(P.BudgetError):
        P.tier_counts(n, 0, 0.3, 0)


def _brute(n, S, b, three):
    s = min(S, n)
    R = n - s
    Br = math.floor(Fraction(str(b)) * 4 * n) - 4 * s
    low = three and Br <= 2 * R
    best = None
    for a in range(R + 1):
        for c in range(R + 1 - a):
            e = R - a - c            # a fp16, c int8, e int4
            if not three and e:
                continue
            if three and low and a:
                continue
            if three and not low and e:
                continue
            cost = 4 * a + 2 * c + e
            if cost > Br:
                continue
            if best is None or cost > best[0]:
                best = (cost, (s + a, c, e))
    return None if best is None else best[1]


def test_brute_force_small():
    grid = [round(0.01 * i, 2) for i in range(0, 101)]
    for n in list(range(0, 25)) + [31, 47, 64]:
        for S in (0, 1, 4):
            for b in grid:
                for three in (1, 0):
                    want = _brute(n, S, b, three)
                    if want is None:
                        with pytest.raises(P.BudgetError):
                            P.tier_counts(n, S, b, three)
                        continue
                    N16, N8, N4, _ = P.tier_counts(n, S, b, three)
                    assert (N16, N8, N4) == want, (n, S, b, three)


def test_budget_rational():
    for n in (1, 7, 256, 1000, 8192, 32768, 65536, 1 << 20):
        for i in range(101):
            b = round(0.01 * i, 2)
            assert P.budget_units(b, n) == math.floor(Fraction(str(b)) * 4 * n)


def test_invariants_random():
    import random
    rnd = random.Random(0)
    for _ in range(3000):
        n = rnd.randint(0, 70000)
        S = rnd.choice([0, 1, 4, 32])
        b = round(rnd.uniform(0, 1), 4)
        three = rnd.choice([0, 1])
        try:
            N16, N8, N4, s = P.tier_counts(n, S, b, three)
        except P.BudgetError:
            continue
        assert N16 + N8 + N4 == n and s == min(S, n) and N16 >= s
        used = 4 * N16 + 2 * N8 + N4
        B = P.budget_units(b, n)
        assert used <= B
        if three and N16 == s:                  # §4.4 branch: exact use
            assert used == B
        elif N16 < n:
            assert B - used in (0, 1)
        if not three:
            assert N4 == 0
        assert not (N16 > s and N4 > 0)         # only adjacent tiers mix


def test_fp16_volume_closed_form():
    # b = 1: every token fp16, payload = §2.1 Bytes_fp16 (no scales)
    for (L, Hq, H, d, n) in [(1, 4, 2, 64, 256), (32, 32, 8, 128, 8192), (3, 4, 1, 256, 17)]:
        pl = P.make_plan(L, Hq, H, d, n, 4, 1.0, 1)
        assert pl.n16 == n and pl.payload_bytes == P.fp16_bytes(L, H, d, n)
        assert P.fp16_bytes(L, H, d, n) == 2 * L * H * d * n * 2


def test_payload_bytes_per_tier():
    pl = P.make_plan(2, 4, 2, 64, 100, 0, 0.3, 1)
    rows = 2 * 2 * 2                        # L * (K,V) * H per token
    assert pl.payload_bytes == rows * (pl.n16 * 128 + pl.n8 * (64 + 2) + pl.n4 * (32 + 2))
    assert pl.off_c16 == 0 <= pl.off_c8 <= pl.off_c4 <= pl.off_s8 <= pl.off_s4 <= pl.payload_bytes


@pytest.mark.parametrize("shape,n,S,b,three,counts,P_bytes", [
    ((1, 4, 2, 64), 256, 4, 0.5, 1, (4, 244, 8), 67552),
    ((32, 32, 8, 128), 8192, 4, 0.5, 1, (4, 8180, 8), 545255424),
    ((28, 28, 4, 128), 32768, 4, 0.6, 0, (6553, 26215, 0), 1139156032),
    ((42, 16, 8, 256), 32768, 4, 0.3, 1, (4, 6541, 26223), 3426269952),
])
def test_workload_plans(shape, n, S, b, three, counts, P_bytes):
    # worked by hand from the closed form for the workload shapes
    pl = P.make_plan(*shape, n, S, b, three)
    assert (pl.n16, pl.n8, pl.n4) == counts
    assert pl.payload_bytes == P_bytes


def test_minima_kv_accounting():
    # Minima-KV page: 18.3 KiB/token over 16 full-attention layers, 4 KV heads,
    # head dim 256, K and V -> about 4.58 bits per scalar, 3.497x vs BF16.
    bps = P.bits_per_scalar(18.3 * 1024, 16, 4, 256, 1)
    assert abs(bps - 4.575) < 1e-9
    assert round(bps, 2) == 4.58 or abs(bps - 4.58) < 0.006
    assert abs(16.0 / bps - 3.497) < 1e-3


def test_domain_errors():
    with pytest.raises(ValueError):
        P.tier_counts(10, 0, 1.5, 1)
    with pytest.raises(ValueError):
        P.tier_counts(10, 0, float("nan"), 1)
    with pytest.raises(P.BudgetError):
        P.tier_counts(1000, 0, 0.2, 1)           # below uniform int4
    with pytest.raises(P.BudgetError):
        P.tier_counts(256, 4, 0.5, 0)            # 2-tier, sinks eat the slack
    with pytest.raises(ValueError):
        P.make_plan(1, 3, 2, 64, 10, 0, 0.5, 1)  # H_q not a multiple of H_kv
    with pytest.raises(ValueError):
        P.make_plan(1, 4, 2, 96, 10, 0, 0.5, 1)  # unsupported head dim


def test_empty_request():
    pl = P.make_plan(2, 4, 2, 64, 0, 4, 0.5, 1)
    assert (pl.n16, pl.n8, pl.n4, pl.payload_bytes) == (0, 0, 0, 0)


# ------------------------------------------------------- overflow modes --
# Reading 4: REJECT (default), DROP (§7.4.3: a 2-tier policy at b = 0.3 sends
# only 60% of the tokens) and FALLBACK (the Korean summary's tier table: the
# lowest band gets int4 if allowed, else int8, whatever the budget).

def test_drop_mode_page_example():
    n = 1000
    N16, N8, N4, s = P.tier_counts(n, 0, 0.3, 0, P.DROP_OVERFLOW)
    assert (N16, N8, N4, s) == (0, 600, 0, 0)             # 60% of the tokens sent
    plan = P.make_plan(1, 4, 2, 64, n, 0, 0.3, 0, P.DROP_OVERFLOW)
    assert plan.n_drop == 400 and plan.used_units <= plan.budget_units


def test_drop_mode_three_tier_and_sinks():
    N16, N8, N4, s = P.tier_counts(1000, 4, 0.2, 1, P.DROP_OVERFLOW)
    # B = 800, sinks take 16, 784 int4 tokens of the 996 others
    assert (N16, N8, N4, s) == (4, 0, 784, 4)
    with pytest.raises(P.BudgetError):                    # the sinks alone overrun
        P.tier_counts(100, 30, 0.2, 1, P.DROP_OVERFLOW)
    # an odd unit left over stays unused in 2-tier
    N16, N8, N4, _ = P.tier_counts(10, 1, 0.33, 0, P.DROP_OVERFLOW)
    assert (N16, N8, N4) == (1, 4, 0)                      # B = 13, Br = 9 -> 4 int8


def test_fallback_mode_overruns():
    N16, N8, N4, s = P.tier_counts(1000, 4, 0.3, 0, P.FALLBACK)
    assert (N16, N8, N4) == (4, 996, 0)
    plan = P.make_plan(2, 4, 2, 64, 1000, 4, 0.3, 0, P.FALLBACK)
    assert plan.used_units == 16 + 2 * 996 > plan.budget_units and plan.n_drop == 0
    N16, N8, N4, s = P.tier_counts(1000, 4, 0.1, 1, P.FALLBACK)
    assert (N16, N8, N4) == (4, 0, 996)


def test_modes_agree_when_the_budget_suffices():
    rng = np.random.default_rng(9)
    for _ in range(300):
        n = int(rng.integers(0, 3000))
        S = int(rng.integers(0, 8))
        b = float(rng.random())
        three = int(rng.integers(0, 2))
        try:
            want = P.tier_counts(n, S, b, three)
        except P.BudgetError:
            continue
        for mode in (P.DROP_OVERFLOW, P.FALLBACK):
            assert P.tier_counts(n, S, b, three, mode) == want
