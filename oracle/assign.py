"""Tier assignment (oracle).

Sources (SpectrumKV paper, arXiv 2606.08635):

* §2.3, Proposition 1 (exchange argument): for fixed tier counts, an optimal
  assignment never gives a lower-precision tier to a more important token.
* §7.4.1 and Algorithm 1: the first S tokens are pinned to fp16 before
  ranking; the remaining tokens are sorted by importance and filled into
  fp16, then int8, then (when allowed) int4.
* The Korean SpectrumKV summary (tier table and quantile thresholds): high /
  mid / low importance go to fp16 / int8 / int4; the first few tokens are
  always fp16.

Readings:

* Ties are broken by position: on equal fp32 scores the lower token index
  ranks higher.
* -0.0 counts as +0.0; scores are non-negative by construction.  NaN or Inf
  scores violate the precondition (asserted here).
* A token's slot is its position among the tokens of the same tier, counted
  in token order (sinks take fp16 slots 0..S'-1).
* map[j] = tier << 30 | slot, tier 0 = fp16, 1 = int8, 2 = int4, 3 = dropped
  (the lowest-ranked tokens when the plan keeps fewer than n, overflow mode
  DROP of the plan oracle).
* order lists the tokens sorted by (tier, token index).

Assignment-only variants (§7 "Baselines", §7.4.1 Table 11, §7.4.2 Table 12):
Random_Tier keeps the tier fractions and ranks by a random key instead of the
importance (the keys are an input: any i.i.d. draw); Balanced spreads each
tier evenly over the positions, ignoring importance.  Reading for Balanced:
the non-sink token at offset r = j - S' gets the key 2^b - 1 - rev_b(r), with
rev_b the reversal of the b low bits and b the fewest bits that hold R - 1,
so the ranking visits positions in van der Corput order and the first k
ranked tokens of any tier boundary are spread evenly over the sequence.
"""

import numpy as np

from .plan import DROP, FP16, INT8, INT4


def assign(score32, n16, n8, n4, sinks):
    """Return (tier[n], slot[n], map[n] uint32, order[n] uint32).

    score32: fp32 scores [n]; n16 includes the sinks; sinks = S'."""
    sc = np.asarray(score32, dtype=np.float32)
    n = sc.shape[0]
    assert n16 + n8 + n4 <= n and 0 <= sinks <= n16
    assert np.all(np.isfinite(sc)), "scores must be finite"
    sc = np.where(sc == 0, np.float32(0.0), sc)          # -0.0 -> +0.0
    tier = np.empty(n, dtype=np.int64)
    tier[:sinks] = FP16
    rest = np.arange(sinks, n)
    # rank the non-sinks by (score descending, index ascending)
    ranked = rest[np.lexsort((rest, -sc[rest].astype(np.float64)))]
    k16 = n16 - sinks
    tier[ranked[:k16]] = FP16
    tier[ranked[k16:k16 + n8]] = INT8
    tier[ranked[k16 + n8:k16 + n8 + n4]] = INT4
    tier[ranked[k16 + n8 + n4:]] = DROP
    slot = np.empty(n, dtype=np.int64)
    for t in (FP16, INT8, INT4, DROP):
        members = np.nonzero(tier == t)[0]                # token order
        slot[members] = np.arange(len(members))
    amap = ((tier << 30) | slot).astype(np.uint32)
    order = np.lexsort((np.arange(n), tier)).astype(np.uint32)
    return tier, slot, amap, order


def weighted_error(score, tier, delta=(0.0, 1.0, 3.0)):
    """Proposition 1's objective sum_j I_j * delta_{tier_j} for a strictly
    increasing per-tier error delta_16 < delta_8 < delta_4."""
    d = np.asarray(delta, dtype=np.float64)
    return float(np.sum(np.asarray(score, dtype=np.float64) * d[np.asarray(tier)]))


def _bitrev(x, b):
    r = 0
    for _ in range(b):
        r = (r << 1) | (x & 1)
        x >>= 1
    return r


def balanced_keys(n, sinks):
    """fp32 keys of the Balanced variant (reading above); sinks get 0."""
    R = n - sinks
    keys = np.zeros(n, dtype=np.float32)
    b = 0
    while (1 << b) < R:
        b += 1
    for r in range(R):
        keys[sinks + r] = np.float32((1 << b) - 1 - _bitrev(r, b))
    return keys
