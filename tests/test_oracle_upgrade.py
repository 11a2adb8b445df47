"""Pins of the cold-tier upgrade oracle (SpectrumKV §4.2 and the cold-tier
fetch paragraph of §8): a hand-written layout example, agreement with the
fp16 segment of the pack oracle, and the round trip that restores the exact
fp16 rows of the upgraded tokens over an int4 transfer."""

import numpy as np

from oracle import assign as OA
from oracle import plan as OP
from oracle import quant as OQ
from oracle import upgrade as OU


def test_layout_hand_example():
    # K[l][j][g][c] = 1000 l + 100 j + 10 g + c, V = -K; L=2, n=3, H=2, d=2
    L, n, H, d = 2, 3, 2, 2
    K = np.zeros((L, n, H, d), dtype=np.float16)
    for l in range(L):
        for j in range(n):
            for g in range(H):
                for c in range(d):
                    K[l, j, g, c] = 1000 * l + 100 * j + 10 * g + c
    V = -K
    got = OU.upgrade_pack(K, V, [2, 0]).view("<f2")
    want = np.array([
        # layer 0, slot 0 = token 2: K heads, then V heads
        200, 201, 210, 211, -200, -201, -210, -211,
        # layer 0, slot 1 = token 0
        0, 1, 10, 11, -0.0, -1, -10, -11,
        # layer 1, slot 0 = token 2
        1200, 1201, 1210, 1211, -1200, -1201, -1210, -1211,
        # layer 1, slot 1 = token 0
        1000, 1001, 1010, 1011, -1000, -1001, -1010, -1011,
    ], dtype=np.float16)
    assert OU.upgrade_bytes(L, H, d, 2) == want.size * 2
    assert np.array_equal(got.view(np.uint16), want.view(np.uint16))


def test_skipped_tokens_leave_payload_bytes():
    K = np.ones((1, 4, 1, 8), dtype=np.float16)
    fill = np.full(OU.upgrade_bytes(1, 1, 8, 3), 0xA5, dtype=np.uint8)
    got = OU.upgrade_pack(K, K, [1, 4, -1], payload=fill).view("<f2").reshape(1, 3, 2, 1, 8)
    assert np.all(got[0, 0] == 1.0)
    assert np.all(got[0, 1:].view(np.uint16) == 0xA5A5)


def test_all_tokens_in_order_equal_the_fp16_segment():
    rng = np.random.default_rng(4)
    L, H, d, n = 2, 3, 64, 37
    K = rng.standard_normal((L, n, H, d)).astype(np.float16)
    V = rng.standard_normal((L, n, H, d)).astype(np.float16)
    plan = OP.make_plan(L, 2 * H, H, d, n, 0, 1.0, 1)           # every token at fp16
    assert plan.n16 == n
    amap = (np.arange(n, dtype=np.uint32))                      # tier 0, slot j
    full = OQ.pack(K, V, amap, plan)
    assert np.array_equal(OU.upgrade_pack(K, V, np.arange(n)), full[:plan.off_c8])


def test_round_trip_restores_fp16_over_int4():
    rng = np.random.default_rng(5)
    L, H, d, n, bs = 2, 2, 64, 50, 16
    K = rng.standard_normal((L, n, H, d)).astype(np.float16)
    V = rng.standard_normal((L, n, H, d)).astype(np.float16)
    plan = OP.make_plan(L, 4, H, d, n, 0, 0.25, 1)             # all int4
    assert plan.n4 == n
    amap = (np.uint32(2) << np.uint32(30)) | np.arange(n, dtype=np.uint32)
    payload = OQ.pack(K, V, amap, plan)
    Kd, Vd = OQ.unpack_dense(payload, amap, plan, L, H, d)
    assert not np.array_equal(Kd, K)                            # int4 is lossy here
    up = np.array([7, 0, 49, 7, 23, 40])
    upl = OU.upgrade_pack(K, V, up)
    OU.upgrade_unpack_dense(upl, up, Kd, Vd)
    Kw, Vw = OQ.unpack_dense(payload, amap, plan, L, H, d)
    for j in range(n):
        src_k, src_v = (K, V) if j in up else (Kw, Vw)
        assert np.array_equal(Kd[:, j].view(np.uint16), src_k[:, j].view(np.uint16)), j
        assert np.array_equal(Vd[:, j].view(np.uint16), src_v[:, j].view(np.uint16)), j
    # paged: same rows through a permuted block table; one block outside the pool
    nb = (n + bs - 1) // bs
    bt = np.array([2, 0, 9, 1], dtype=np.int32)[:nb]            # block 9 does not exist
    kc = np.zeros((L, 3, bs, H, d), dtype=np.float16)
    vc = np.zeros_like(kc)
    OU.upgrade_unpack_paged(upl, up, n, bt, kc, vc, bs)
    assert np.array_equal(kc[:, 2, 7], K[:, 7]) and np.array_equal(vc[:, 2, 0], V[:, 0])
    assert np.array_equal(kc[:, 1, 49 % bs], K[:, 49]) and np.array_equal(vc[:, 0, 7], V[:, 23])
    # token 40 sits in block 9, outside the pool: nothing else was written
    assert np.count_nonzero(kc) == np.count_nonzero(K[:, [7, 0, 49, 23]])
    assert np.count_nonzero(vc) == np.count_nonzero(V[:, [7, 0, 49, 23]])
