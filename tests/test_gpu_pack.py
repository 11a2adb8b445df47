"""GPU parity of pack and unpack (dense and paged) against the oracle:
payload bytes, codes, scales and dequantized fp16 KV must be bit-exact when
the map comes from the oracle's assignment."""

import numpy as np
import pytest
import torch

from oracle import assign as OA
from oracle import plan as OP
from oracle import quant as OQ
import serving_sk_score_amd as sk
from workloads import gen, get_config
from tests.gpu_helpers import Guarded, fill_layers, make_kv, make_kv_deep, say, tied_scores, to_dev

pytestmark = pytest.mark.gpu

CASES = [
    # L, Hq, H, d, n, S, b, three
    (1, 4, 2, 64, 256, 4, 0.5, 1),       # tiny shape: 4 fp16, 244 int8, 8 int4
    (2, 8, 4, 128, 1000, 4, 0.45, 1),    # int8 + int4 + sinks
    (3, 4, 1, 256, 77, 4, 0.7, 1),       # fp16 + int8, single KV head
    (2, 14, 2, 128, 513, 4, 0.6, 0),     # 2-tier
    (1, 2, 2, 64, 1, 0, 1.0, 1),         # one token
    (2, 4, 2, 64, 5, 4, 1.0, 1),         # n close to S
    (2, 8, 8, 256, 333, 0, 0.25, 1),     # all int4
    (1, 32, 8, 128, 1025, 4, 0.3, 1),    # Mistral heads, ragged n
]


def _oracle_map(pl, n, seed):
    s = tied_scores(seed, n)
    _, _, amap, order = OA.assign(s, pl.n16, pl.n8, pl.n4, pl.sinks)
    return amap, order


def _run(L, Hq, H, d, n, S, b, three, seed=0, kv=make_kv):
    say("pack/unpack", dict(L=L, Hq=Hq, H=H, d=d, n=n, S=S, b=b, three=three))
    shape = sk.Shape(L, Hq, H, d)
    pl = sk.plan_make(shape, sk.Policy(n, S, three, b))
    opl = OP.make_plan(L, Hq, H, d, n, S, b, three)
    K, V = kv(seed + n, L, n, H, d)
    amap, order = _oracle_map(opl, n, seed)
    want = OQ.pack(K, V, amap, opl)
    Kd, Vd = to_dev(K), to_dev(V)
    md, od = to_dev(amap.view(np.int32)), to_dev(order.view(np.int32))
    buf = Guarded(pl.payload_bytes)
    sk.pack(shape, pl, Kd, Vd, md, od, buf.bytes)
    torch.cuda.synchronize()
    buf.check()
    got = buf.bytes.cpu().numpy()
    assert got.size == want.size
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, f"{bad.size} payload bytes differ, first at {bad[:5]}"
    # determinism
    buf2 = Guarded(pl.payload_bytes, fill=0x5A)
    sk.pack(shape, pl, Kd, Vd, md, od, buf2.bytes)
    torch.cuda.synchronize()
    assert torch.equal(buf.bytes, buf2.bytes)
    # dense unpack
    Kw, Vw = OQ.unpack_dense(want, amap, opl, L, H, d)
    ko = Guarded(K.nbytes)
    vo = Guarded(V.nbytes)
    sk.unpack(shape, pl, buf.bytes, md, ko.as_(torch.float16, K.shape), vo.as_(torch.float16, V.shape))
    torch.cuda.synchronize()
    ko.check()
    vo.check()
    assert np.array_equal(ko.as_(torch.int16, K.shape).cpu().numpy(), Kw.view(np.int16))
    assert np.array_equal(vo.as_(torch.int16, V.shape).cpu().numpy(), Vw.view(np.int16))
    # paged unpack through a permuted block table, with spare blocks
    bs = 16
    nb = (n + bs - 1) // bs
    total = nb + 5
    rng = np.random.default_rng(seed + 7)
    bt = rng.permutation(total)[:nb].astype(np.int32)
    cshape = (L, total, bs, H, d)
    kc = torch.full(cshape, 3.0, dtype=torch.float16, device="cuda")
    vc = torch.full(cshape, 3.0, dtype=torch.float16, device="cuda")
    sk.unpack_paged(shape, pl, buf.bytes, md, kc, vc, to_dev(bt), bs)
    torch.cuda.synchronize()
    kcw = np.full(cshape, 3.0, dtype=np.float16)
    vcw = np.full(cshape, 3.0, dtype=np.float16)
    OQ.unpack_paged(want, amap, opl, L, H, d, bt, kcw, vcw, bs)
    assert np.array_equal(kc.cpu().numpy().view(np.int16), kcw.view(np.int16))
    assert np.array_equal(vc.cpu().numpy().view(np.int16), vcw.view(np.int16))


@pytest.mark.parametrize("case", CASES, ids=lambda c: "L%d_Hq%d_H%d_d%d_n%d_S%d_b%s_t%d" % c)
def test_pack_unpack_bitexact(case):
    _run(*case)


def test_pack_unpack_at_layer_limit():
    """65,535 layers, the most a shape admits (the layer is the second
    dimension of every pack and unpack grid): fp16 sinks, int8 and int4 rows
    of an 11-token request, bit-exact through pack, dense and paged unpack."""
    _run(65535, 4, 2, 64, 11, 2, 0.55, 1, kv=make_kv_deep)


def test_paged_skips_out_of_range_blocks():
    L, Hq, H, d, n, S, b, three = 1, 4, 2, 64, 40, 4, 0.5, 1
    say("paged bounds check", n)
    shape = sk.Shape(L, Hq, H, d)
    pl = sk.plan_make(shape, sk.Policy(n, S, three, b))
    opl = OP.make_plan(L, Hq, H, d, n, S, b, three)
    K, V = make_kv(5, L, n, H, d)
    amap, order = _oracle_map(opl, n, 5)
    payload = torch.empty(pl.payload_bytes, dtype=torch.uint8, device="cuda")
    md = to_dev(amap.view(np.int32))
    sk.pack(shape, pl, to_dev(K), to_dev(V), md, None, payload)
    bt = np.array([0, 7, 2], dtype=np.int32)        # block 7 does not exist (num_blocks = 3)
    kc = torch.zeros((L, 3, 16, H, d), dtype=torch.float16, device="cuda")
    vc = torch.zeros_like(kc)
    sk.unpack_paged(shape, pl, payload, md, kc, vc, to_dev(bt), 16)
    torch.cuda.synchronize()
    assert torch.count_nonzero(kc[:, 1]) == 0                      # untouched
    Kw, _ = OQ.unpack_dense(OQ.pack(K, V, amap, opl), amap, opl, L, H, d)
    assert np.array_equal(kc[0, 0].cpu().numpy().view(np.int16), Kw[0, :16].view(np.int16))
    assert np.array_equal(kc[0, 2, :8].cpu().numpy().view(np.int16), Kw[0, 32:40].view(np.int16))


@pytest.mark.parametrize("name", ["mistral7b", "qwen25_7b_2tier", "gemma2_9b"])
def test_full_size_sampled_layers(name):
    """Full workload size, the launch configuration the benchmark times; the
    oracle checks whole sampled layers of the payload and of the unpack."""
    cfg = get_config(name)
    L, Hq, H, d, n = cfg.layers, cfg.q_heads, cfg.kv_heads, cfg.head_dim, cfg.tokens
    say("full-size pack", name)
    shape = sk.Shape(L, Hq, H, d)
    pl = sk.plan_make(shape, sk.Policy(n, cfg.sinks, cfg.three_tier, cfg.budget))
    opl = OP.make_plan(L, Hq, H, d, n, cfg.sinks, cfg.budget, cfg.three_tier)
    amap, order = _oracle_map(opl, n, 11)
    md = to_dev(amap.view(np.int32))
    Kd = torch.empty((L, n, H, d), dtype=torch.float16, device="cuda")
    Vd = torch.empty_like(Kd)
    layers = sorted({0, L - 1, L // 2})
    hk = fill_layers(cfg, gen.keys, Kd, keep=layers)
    hv = fill_layers(cfg, gen.values, Vd, keep=layers)
    say("inputs resident", name)
    payload = Guarded(pl.payload_bytes)
    sk.pack(shape, pl, Kd, Vd, md, None, payload.bytes)
    Ko = torch.empty_like(Kd)
    Vo = torch.empty_like(Vd)
    sk.unpack(shape, pl, payload.bytes, md, Ko, Vo)
    torch.cuda.synchronize()
    payload.check()
    say("checking layers", layers)
    got = payload.bytes.cpu().numpy()
    for layer in layers:
        k, v = hk[layer], hv[layer]
        for off, data in OQ.pack_layer(k, v, layer, amap, opl):
            assert np.array_equal(got[off:off + data.size], data), (name, layer, off)
        kw, vw = OQ.unpack_layer(got, layer, amap, opl, H, d)
        assert np.array_equal(Ko[layer].cpu().numpy().view(np.int16), kw.view(np.int16))
        assert np.array_equal(Vo[layer].cpu().numpy().view(np.int16), vw.view(np.int16))


def _every_scale_rows(qmax, d, seed):
    """One row per non-negative finite fp16 absmax (31,744 rows): row r has
    max |x| = the fp16 with bits r, placed at a random element with a random
    sign, so every scale the quantizer can produce (fp16 subnormal scales,
    underflow to 0, the largest) occurs; the other elements are uniform in
    [-a, a] with a quarter of them at the half-steps (k + 1/2) s, where the
    rounding of the code is decided by the last bit of the quotient."""
    rng = np.random.default_rng(seed)
    a = np.arange(0x7C00, dtype=np.uint16).view(np.float16).astype(np.float32)
    rows = a.size
    s = (a / np.float32(qmax)).astype(np.float16).astype(np.float32)
    x = rng.uniform(-1.0, 1.0, (rows, d)).astype(np.float32) * a[:, None]
    k = rng.integers(-qmax, qmax, size=(rows, d)).astype(np.float32)
    half = (k + np.float32(0.5)) * s[:, None]
    tie = rng.random((rows, d)) < 0.25
    x = np.where(tie, np.clip(half, -a[:, None], a[:, None]), x)
    x = x.astype(np.float16)
    at = rng.integers(0, d, size=rows)
    sign = rng.choice(np.array([-1.0, 1.0], dtype=np.float32), size=rows)
    x[np.arange(rows), at] = (sign * a).astype(np.float16)
    return x


@pytest.mark.parametrize("qmax,b,d", [(127, 0.5, 128), (7, 0.25, 128), (127, 0.5, 64), (7, 0.25, 256)])
def test_every_fp16_scale(qmax, b, d):
    """Every tier-row absmax an fp16 row can have, all tokens in one
    quantized tier: payload bytes and dequantized KV bit-exact against the
    oracle."""
    H = 2
    rows = _every_scale_rows(qmax, d, seed=qmax * 1000 + d)
    n = rows.shape[0] // (2 * H)
    say("every fp16 scale", dict(qmax=qmax, d=d, n=n))
    K = np.ascontiguousarray(rows[: n * H].reshape(1, n, H, d))
    V = np.ascontiguousarray(rows[n * H:].reshape(1, n, H, d))
    shape = sk.Shape(1, 4, H, d)
    pl = sk.plan_make(shape, sk.Policy(n, 0, 1, b))
    opl = OP.make_plan(1, 4, H, d, n, 0, b, 1)
    assert (opl.n8, opl.n4) == ((n, 0) if qmax == 127 else (0, n))
    amap, _ = _oracle_map(opl, n, 3)
    want = OQ.pack(K, V, amap, opl)
    Kd, Vd = to_dev(K), to_dev(V)
    md = to_dev(amap.view(np.int32))
    buf = Guarded(pl.payload_bytes)
    sk.pack(shape, pl, Kd, Vd, md, None, buf.bytes)
    torch.cuda.synchronize()
    buf.check()
    got = buf.bytes.cpu().numpy()
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, f"{bad.size} payload bytes differ, first at {bad[:5]}"
    Kw, Vw = OQ.unpack_dense(want, amap, opl, 1, H, d)
    Ko = torch.empty_like(Kd)
    Vo = torch.empty_like(Vd)
    sk.unpack(shape, pl, buf.bytes, md, Ko, Vo)
    torch.cuda.synchronize()
    assert np.array_equal(Ko.cpu().numpy().view(np.int16), Kw.view(np.int16))
    assert np.array_equal(Vo.cpu().numpy().view(np.int16), Vw.view(np.int16))
