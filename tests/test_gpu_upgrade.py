"""GPU parity of the cold-tier upgrade (SpectrumKV §4.2 and the cold-tier fetch
paragraph of §8) against the oracle, bit for bit: the upgrade payload, the
dense KV after a transfer followed by an upgrade, and the paged cache."""

import numpy as np
import pytest
import torch

from oracle import assign as OA
from oracle import plan as OP
from oracle import quant as OQ
from oracle import upgrade as OU
import serving_sk_score_amd as sk
from workloads import gen, get_config
from tests.gpu_helpers import FILL, Guarded, make_kv, say, tied_scores, to_dev

pytestmark = pytest.mark.gpu

CASES = [
    # L, Hq, H, d, n, m
    (1, 4, 2, 64, 256, 10),
    (2, 8, 4, 128, 1000, 77),
    (3, 4, 1, 256, 77, 5),
    (2, 14, 2, 128, 513, 1),
    (1, 32, 8, 128, 1025, 100),
]


def _token_list(rng, n, m):
    """m entries: mostly distinct tokens, a repeat, and (when m > 2) one entry
    outside [0, n) and one that is 2^32 - 1 as a u32."""
    t = rng.choice(n, size=m, replace=False).astype(np.int64)
    if m > 2:
        t[1] = t[0]
        t[2] = n + 5
    if m > 4:
        t[4] = 0xFFFFFFFF
    return t


def _u32_dev(t):
    return to_dev(np.asarray(t, dtype=np.uint32).view(np.int32))


@pytest.mark.parametrize("case", CASES, ids=lambda c: "L%d_Hq%d_H%d_d%d_n%d_m%d" % c)
def test_upgrade_after_transfer(case):
    L, Hq, H, d, n, m = case
    say("upgrade", case)
    rng = np.random.default_rng(n + m)
    shape = sk.Shape(L, Hq, H, d)
    K, V = make_kv(900 + n, L, n, H, d)
    Kd, Vd = to_dev(K), to_dev(V)
    tokens = _token_list(rng, n, m)
    td = _u32_dev(tokens)

    # upgrade payload: skipped entries keep the canary bytes
    size = sk.upgrade_bytes(shape, m)
    assert size == OU.upgrade_bytes(L, H, d, m)
    buf = Guarded(size)
    sk.upgrade_pack(shape, Kd, Vd, td, buf.bytes)
    torch.cuda.synchronize()
    buf.check()
    want_up = OU.upgrade_pack(K, V, tokens, payload=np.full(size, FILL, dtype=np.uint8))
    got_up = buf.bytes.cpu().numpy()
    bad = np.nonzero(got_up != want_up)[0]
    assert bad.size == 0, f"{bad.size} upgrade payload bytes differ, first at {bad[:5]}"

    # a 3-tier transfer at b = 0.3 (int8 + int4), dense unpack, then the upgrade
    pol = sk.Policy(n, 4, 1, 0.3)
    pl = sk.plan_make(shape, pol)
    opl = OP.make_plan(L, Hq, H, d, n, 4, 0.3, 1)
    _, _, amap, _ = OA.assign(tied_scores(n, n), opl.n16, opl.n8, opl.n4, opl.sinks)
    md = to_dev(amap.view(np.int32))
    payload = torch.empty(pl.payload_bytes, dtype=torch.uint8, device="cuda")
    sk.pack(shape, pl, Kd, Vd, md, None, payload)
    Ko = torch.empty_like(Kd)
    Vo = torch.empty_like(Vd)
    sk.unpack(shape, pl, payload, md, Ko, Vo)
    sk.upgrade_unpack(shape, n, buf.bytes, td, Ko, Vo)
    torch.cuda.synchronize()
    Kw, Vw = OQ.unpack_dense(OQ.pack(K, V, amap, opl), amap, opl, L, H, d)
    OU.upgrade_unpack_dense(want_up, tokens, Kw, Vw)
    assert np.array_equal(Ko.cpu().numpy().view(np.int16), Kw.view(np.int16))
    assert np.array_equal(Vo.cpu().numpy().view(np.int16), Vw.view(np.int16))
    live = tokens[tokens < n]
    assert np.array_equal(Kw[:, live], K[:, live])           # upgraded rows are exact

    # paged: permuted pool with spare blocks and one id outside the pool
    bs = 16
    nb = (n + bs - 1) // bs
    total = nb + 3
    bt = rng.permutation(total)[:nb].astype(np.int32)
    if nb > 1:
        bt[nb // 2] = total + 7
    cshape = (L, total, bs, H, d)
    kc = torch.full(cshape, 0, dtype=torch.int16, device="cuda").fill_(0x4248).view(torch.float16)
    vc = torch.full(cshape, 0, dtype=torch.int16, device="cuda").fill_(0x4248).view(torch.float16)
    sk.upgrade_unpack_paged(shape, n, buf.bytes, td, kc, vc, to_dev(bt), bs)
    torch.cuda.synchronize()
    kcw = np.full(cshape, 0x4248, dtype=np.int16).view(np.float16)
    vcw = np.full(cshape, 0x4248, dtype=np.int16).view(np.float16)
    OU.upgrade_unpack_paged(want_up, tokens, n, bt, kcw, vcw, bs)
    assert np.array_equal(kc.cpu().numpy().view(np.int16), kcw.view(np.int16))
    assert np.array_equal(vc.cpu().numpy().view(np.int16), vcw.view(np.int16))


def test_upgrade_full_size_sampled_layers():
    """Mistral-7B shape at full length with 1024 upgraded tokens (the launch
    configuration the benchmark times); sampled layers checked whole."""
    cfg = get_config("mistral7b")
    L, Hq, H, d, n = cfg.layers, cfg.q_heads, cfg.kv_heads, cfg.head_dim, cfg.tokens
    m = n // 8
    say("full-size upgrade", n, m)
    shape = sk.Shape(L, Hq, H, d)
    tokens = np.random.default_rng(8).choice(n, size=m, replace=False)
    td = _u32_dev(tokens)
    layers = sorted({0, L // 2, L - 1})
    Kd = torch.empty((L, n, H, d), dtype=torch.float16, device="cuda")
    Vd = torch.empty_like(Kd)
    hk, hv = {}, {}
    for layer in range(L):
        k, v = gen.keys(cfg, layer), gen.values(cfg, layer)
        Kd[layer].copy_(torch.from_numpy(k))
        Vd[layer].copy_(torch.from_numpy(v))
        if layer in layers:
            hk[layer], hv[layer] = k, v
    up = Guarded(sk.upgrade_bytes(shape, m))
    sk.upgrade_pack(shape, Kd, Vd, td, up.bytes)
    bs = 16
    nb = (n + bs - 1) // bs
    bt = np.random.default_rng(0).permutation(nb).astype(np.int32)
    kc = torch.zeros((L, nb, bs, H, d), dtype=torch.float16, device="cuda")
    vc = torch.zeros_like(kc)
    sk.upgrade_unpack_paged(shape, n, up.bytes, td, kc, vc, to_dev(bt), bs)
    torch.cuda.synchronize()
    up.check()
    rows = up.bytes.cpu().numpy().view("<f2").reshape(L, m, 2, H, d)
    for layer in layers:
        k, v = hk[layer], hv[layer]
        assert np.array_equal(rows[layer, :, 0].view(np.int16), k[tokens].view(np.int16))
        assert np.array_equal(rows[layer, :, 1].view(np.int16), v[tokens].view(np.int16))
        blk, pos = bt[tokens // bs], tokens % bs
        kl = kc[layer].cpu().numpy()
        vl = vc[layer].cpu().numpy()
        assert np.array_equal(kl[blk, pos].view(np.int16), k[tokens].view(np.int16))
        assert np.array_equal(vl[blk, pos].view(np.int16), v[tokens].view(np.int16))
        mask = np.ones((nb, bs), dtype=bool)
        mask[blk, pos] = False
        assert not kl[mask].any() and not vl[mask].any()       # nothing else written
