"""GPU parity of the policy variants against the oracle, bit for bit: budget
overflow by dropping (SpectrumKV §7.4.3) or by falling back to the cheapest
tier (the Korean summary's tier table), the Balanced ranking keys (§7.4.1
Table 11) and Random_Tier (§7 baselines, Table 12: the ranked assignment on
random keys) - the tier map, the order, the payload and the dense and paged
unpack, where dropped tokens' rows must stay untouched."""

import numpy as np
import pytest
import torch

from oracle import assign as OA
from oracle import plan as OP
from oracle import quant as OQ
import serving_sk_score_amd as sk
from tests.gpu_helpers import Guarded, make_kv, say, tied_scores, to_dev, u32

pytestmark = pytest.mark.gpu

CANARY = 0x4248


def _round_trip(L, Hq, H, d, n, S, b, three, mode, keys):
    shape = sk.Shape(L, Hq, H, d)
    pol = sk.Policy(n, S, three, b, mode)
    pl = sk.plan_make(shape, pol)
    opl = OP.make_plan(L, Hq, H, d, n, S, b, three, mode)
    assert (pl.n16, pl.n8, pl.n4, pl.n_drop) == (opl.n16, opl.n8, opl.n4, opl.n_drop)
    kd = to_dev(keys)
    amap = torch.empty(n, dtype=torch.int32, device="cuda")
    order = torch.empty(n, dtype=torch.int32, device="cuda")
    sk.assign_tiers(pol, pl, kd, amap, order)
    torch.cuda.synchronize()
    _, _, want_map, want_order = OA.assign(keys, opl.n16, opl.n8, opl.n4, opl.sinks)
    assert np.array_equal(u32(amap), want_map)
    assert np.array_equal(u32(order), want_order)
    K, V = make_kv(70 + n, L, n, H, d)
    Kd, Vd = to_dev(K), to_dev(V)
    buf = Guarded(max(pl.payload_bytes, 1))
    payload = buf.bytes[:pl.payload_bytes]
    sk.pack(shape, pl, Kd, Vd, amap, order, payload)
    torch.cuda.synchronize()
    buf.check()
    want = OQ.pack(K, V, want_map, opl)
    assert np.array_equal(payload.cpu().numpy(), want)
    # dense: dropped tokens keep the canary
    Ko = torch.full(K.shape, 0, dtype=torch.int16, device="cuda").fill_(CANARY).view(torch.float16)
    Vo = torch.full(K.shape, 0, dtype=torch.int16, device="cuda").fill_(CANARY).view(torch.float16)
    sk.unpack(shape, pl, payload, amap, Ko, Vo)
    Kw = np.full(K.shape, CANARY, dtype=np.int16).view(np.float16)
    Vw = np.full(K.shape, CANARY, dtype=np.int16).view(np.float16)
    OQ.unpack_dense(want, want_map, opl, L, H, d, Kw, Vw)
    # paged through a permuted pool
    bs = 16
    nb = (n + bs - 1) // bs
    bt = np.random.default_rng(n).permutation(nb + 2)[:nb].astype(np.int32)
    cshape = (L, nb + 2, bs, H, d)
    kc = torch.full(cshape, 0, dtype=torch.int16, device="cuda").fill_(CANARY).view(torch.float16)
    vc = torch.full(cshape, 0, dtype=torch.int16, device="cuda").fill_(CANARY).view(torch.float16)
    sk.unpack_paged(shape, pl, payload, amap, kc, vc, to_dev(bt), bs)
    torch.cuda.synchronize()
    assert np.array_equal(Ko.cpu().numpy().view(np.int16), Kw.view(np.int16))
    assert np.array_equal(Vo.cpu().numpy().view(np.int16), Vw.view(np.int16))
    kcw = np.full(cshape, CANARY, dtype=np.int16).view(np.float16)
    vcw = np.full(cshape, CANARY, dtype=np.int16).view(np.float16)
    OQ.unpack_paged(want, want_map, opl, L, H, d, bt, kcw, vcw, bs)
    assert np.array_equal(kc.cpu().numpy().view(np.int16), kcw.view(np.int16))
    assert np.array_equal(vc.cpu().numpy().view(np.int16), vcw.view(np.int16))
    return pl


OVERFLOW_CASES = [
    # L, Hq, H, d, n, S, b, three, mode
    (2, 8, 4, 128, 1000, 4, 0.3, 0, sk.OVERFLOW_DROP),       # the page's 60% case
    (1, 4, 2, 64, 257, 0, 0.2, 1, sk.OVERFLOW_DROP),         # int4 + dropped
    (1, 32, 8, 128, 8192, 4, 0.45, 0, sk.OVERFLOW_DROP),     # Mistral heads, one layer
    (2, 8, 4, 128, 1000, 4, 0.3, 0, sk.OVERFLOW_FALLBACK),   # all int8, over budget
    (1, 4, 1, 256, 99, 4, 0.1, 1, sk.OVERFLOW_FALLBACK),     # all int4, over budget
]


@pytest.mark.parametrize("case", OVERFLOW_CASES,
                         ids=lambda c: "L%d_Hq%d_H%d_d%d_n%d_S%d_b%s_t%d_mode%d" % c)
def test_budget_overflow(case):
    say("overflow", case)
    L, Hq, H, d, n, S, b, three, mode = case
    pl = _round_trip(*case, keys=tied_scores(n + 3, n))
    if mode == sk.OVERFLOW_DROP:
        assert pl.n_drop > 0 and pl.used_units <= pl.budget_units
    else:
        assert pl.n_drop == 0 and pl.used_units > pl.budget_units


@pytest.mark.parametrize("n,S", [(1, 0), (2, 0), (5, 4), (300, 4), (1027, 0), (65536, 4)])
def test_balanced_keys(n, S):
    say("balanced keys", n, S)
    out = Guarded(4 * n)
    keys = out.as_(torch.float32, (n,))
    sk.balanced_keys(n, S, keys)
    torch.cuda.synchronize()
    out.check()
    want = OA.balanced_keys(n, min(S, n))
    assert np.array_equal(keys.cpu().numpy().view(np.uint32), want.view(np.uint32))


def test_balanced_and_random_tier_assignment():
    L, Hq, H, d, n, S, b = 2, 8, 4, 128, 1000, 4, 0.35
    say("balanced round trip")
    _round_trip(L, Hq, H, d, n, S, b, 1, sk.OVERFLOW_REJECT,
                keys=OA.balanced_keys(n, S))
    say("random-tier round trip")
    rkeys = np.random.default_rng(31).random(n).astype(np.float32)
    pl = _round_trip(L, Hq, H, d, n, S, b, 1, sk.OVERFLOW_REJECT, keys=rkeys)
    # the same tier fractions as the importance-ranked policy
    greedy = sk.plan_make(sk.Shape(L, Hq, H, d), sk.Policy(n, S, 1, b))
    assert pl.counts() == greedy.counts()
