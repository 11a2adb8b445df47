"""Budget -> tier counts, payload size and payload layout (oracle).

Sources (SpectrumKV paper, arXiv 2606.08635):

* §2.1, KV transfer budget: the fp16 KV volume is 2 L H_kv d_h n s16 bytes and
  the normalized tier costs are c(16)=1, c(8)=1/2, c(4)=1/4.
* §4.4, budget-to-tier mapping: with f16 = 0, f8 = 4b - 1 and f4 = 2 - 4b
  (so that f8/2 + f4/4 = b and f8 + f4 = 1).
* §7.4.1 and Algorithm 1: the first S tokens are pinned to fp16 before the
  ranking; the rest are allocated fp16 / int8 / optionally int4 under the
  normalized budget.
* §4.5 and §7.4.3: the 2-tier (fp16 + int8) fallback when int4 is not allowed.

Readings where the pages leave a step open:

1. Budget units are quarter tokens (fp16 = 4, int8 = 2, int4 = 1).  The whole
   budget is B = floor(4 b n + 1e-7), evaluated in float64.
2. Sinks are paid out of the budget first: Br = B - 4 S', S' = min(S, n).
3. The remaining R = n - S' tokens follow §4.4 with b' = Br / (4R): for
   Br <= 2R the int8/int4 split is exact (n8 = Br - R, n4 = 2R - Br); the page
   prints the mapping only for b <= 1/2, so above it the same linear rule is
   extended to fp16/int8 (n16 = floor((Br - 2R)/2), n8 = R - n16), capped at
   n16 = R.
4. A budget that cannot pay the cheapest allowed representation of every
   token (3-tier: Br < R; 2-tier: Br < 2R) is rejected, never overrun, in
   the default overflow mode REJECT.  Two other modes follow the pages'
   other statements about that case:
   - DROP (§7.4.3: at b = 0.3 a 2-tier policy can send only 60% of the
     tokens, the rest are dropped): as many remaining tokens as Br pays at
     the cheapest allowed tier are kept, floor(Br / cost); the lowest-ranked
     rest are dropped (no bytes).  The sinks must still be paid (Br >= 0).
   - FALLBACK (the Korean summary's tier table: below the low quantile a
     token gets int4 when allowed, otherwise int8): every remaining token
     goes at the cheapest allowed tier and the budget is overrun.
5. Scale bytes are not charged to the budget (§2.1 uses nominal costs); they
   appear in the payload byte count.
6. Payload layout (the pages define none): five segments
   c16 | c8 | c4 | s8 | s4, each row-major over [layer][slot][K|V][kv head]
   (codes additionally over the d elements), fp16 scales, no padding.
"""

import math
from dataclasses import dataclass

FP16, INT8, INT4 = 0, 1, 2
DROP = 3                                     # a dropped token: not sent
REJECT, DROP_OVERFLOW, FALLBACK = 0, 1, 2    # budget overflow modes (reading 4)
UNITS = {FP16: 4, INT8: 2, INT4: 1}          # §2.1 costs in quarter tokens


class BudgetError(ValueError):
    """The budget cannot pay for every token at the cheapest allowed tier."""


@dataclass(frozen=True)
class Plan:
    n16: int            # fp16 tokens, sinks included
    n8: int
    n4: int
    sinks: int          # S' = min(S, n)
    budget_units: int   # B
    used_units: int     # 4 N16 + 2 N8 + N4
    payload_bytes: int
    off_c16: int
    off_c8: int
    off_c4: int
    off_s8: int
    off_s4: int
    n_drop: int = 0     # tokens sent nowhere (overflow mode DROP)


def fp16_bytes(L, H_kv, d, n):
    """§2.1: Bytes_fp16(n) = 2 L H_kv d_h n s16, with s16 = 2 bytes."""
    return 2 * L * H_kv * d * n * 2


def budget_units(b, n):
    """Reading 1: B = floor(4 b n + 1e-7) in float64 (quarter-token units)."""
    return int(math.floor(4.0 * float(b) * float(n) + 1e-7))


def tier_counts(n, S, b, three_tier, overflow=REJECT):
    """Return (N16, N8, N4, S') for one request (§4.4, §7.4.1, Algorithm 1);
    n - N16 - N8 - N4 tokens are dropped (only in overflow mode DROP)."""
    if n < 0 or S < 0:
        raise ValueError("n and S must be non-negative")
    if not (math.isfinite(b) and 0.0 <= b <= 1.0):
        raise ValueError("the budget b is a fraction of the fp16 bytes, 0 <= b <= 1")
    if overflow not in (REJECT, DROP_OVERFLOW, FALLBACK):
        raise ValueError("unknown overflow mode")
    s = min(S, n)
    R = n - s
    Br = budget_units(b, n) - 4 * s
    cheapest = UNITS[INT4] if three_tier else UNITS[INT8]
    if Br < cheapest * R and overflow != REJECT:
        if overflow == FALLBACK:
            kept = R
        else:
            if Br < 0:
                raise BudgetError(f"budget pays {Br} quarter units after the sinks")
            kept = Br // cheapest
        return (s, 0, kept, s) if three_tier else (s, kept, 0, s)
    if three_tier:
        if Br < R:
            raise BudgetError(f"budget pays {Br} quarter units for {R} tokens")
        if Br <= 2 * R:                           # §4.4: int8 + int4 only
            n16, n8, n4 = 0, Br - R, 2 * R - Br
        else:                                     # reading 3: fp16 + int8
            n16 = min(R, (Br - 2 * R) // 2)
            n8, n4 = R - n16, 0
    else:
        if Br < 2 * R:
            raise BudgetError(f"2-tier budget pays {Br} quarter units for {R} tokens")
        n16 = min(R, (Br - 2 * R) // 2)
        n8, n4 = R - n16, 0
    return s + n16, n8, n4, s


def make_plan(L, H_q, H_kv, d, n, S, b, three_tier, overflow=REJECT):
    """Counts plus the byte layout of the payload (reading 6)."""
    if d not in (64, 128, 256) or H_kv <= 0 or H_q % H_kv or L <= 0:
        raise ValueError("unsupported shape")
    N16, N8, N4, s = tier_counts(n, S, b, three_tier, overflow)
    rows16 = L * N16 * 2 * H_kv      # (layer, slot, K|V, head) rows per tier
    rows8 = L * N8 * 2 * H_kv
    rows4 = L * N4 * 2 * H_kv
    off_c16 = 0
    off_c8 = off_c16 + rows16 * d * 2
    off_c4 = off_c8 + rows8 * d
    off_s8 = off_c4 + rows4 * (d // 2)
    off_s4 = off_s8 + rows8 * 2
    total = off_s4 + rows4 * 2
    return Plan(n16=N16, n8=N8, n4=N4, sinks=s,
                budget_units=budget_units(b, n),
                used_units=4 * N16 + 2 * N8 + N4,
                payload_bytes=total, off_c16=off_c16, off_c8=off_c8,
                off_c4=off_c4, off_s8=off_s8, off_s4=off_s4,
                n_drop=n - N16 - N8 - N4)


def bits_per_scalar(payload_bytes, L, H_kv, d, n):
    """Transferred bits per K/V scalar, scales included (the accounting used
    for effective rates on the Minima-KV page)."""
    return payload_bytes * 8.0 / (2 * L * H_kv * d * n)
