"""GPU parity of decode attention straight from the payload (SpectrumKV §4.2)
against the float64 oracle on the dequantized rows.

Tolerance, from the kernel's arithmetic: q.k and p.v accumulate in fp32 from
exact fp16 products, and each probability is rounded to fp16 once (relative
error <= 2^-11, used in numerator and denominator alike), so the output is a
convex combination whose weights are off by at most ~2^-10 relative:
|o - o_ref| <= 1e-3 * max|v_hat| over the (layer, KV head), and
|lse - lse_ref| <= 1e-3."""

import numpy as np
import pytest
import torch

from oracle import assign as OA
from oracle import decode as OD
from oracle import plan as OP
from oracle import quant as OQ
import serving_sk_score_amd as sk
from workloads import gen, get_config
from tests.gpu_helpers import Guarded, make_kv, make_kv_deep, say, tied_scores, to_dev

pytestmark = pytest.mark.gpu

TOL = 1e-3


def _check(o, lse, want_o, want_lse, vmax, tag):
    for li in range(o.shape[0]):
        for h in range(o.shape[1]):
            err = np.abs(o[li, h].astype(np.float64) - want_o[li, h]).max()
            assert err <= TOL * vmax[li, h], f"{tag} layer {li} head {h}: {err:.3g} > {TOL * vmax[li, h]:.3g}"
    if lse is not None:
        fin = np.isfinite(want_lse)
        assert np.array_equal(np.isfinite(lse), fin), tag
        assert np.abs(lse[fin] - want_lse[fin]).max(initial=0.0) <= TOL, tag


def _vmax(payload, amap, plan, layers, H, d, Hq):
    out = np.zeros((len(layers), Hq))
    sent = (amap >> 30) <= 2
    for i, layer in enumerate(layers):
        _, v = OQ.unpack_layer(payload, layer, amap, plan, H, d)
        for h in range(Hq):
            g = h // (Hq // H)
            out[i, h] = np.abs(v[sent, g].astype(np.float64)).max(initial=1e-30)
    return out


CASES = [
    # L, Hq, H, d, n, S, b, three, overflow
    (1, 4, 2, 64, 256, 4, 0.5, 1, 0),        # tiny shape
    (2, 8, 4, 128, 1000, 4, 0.3, 1, 0),      # mostly int4
    (2, 14, 2, 128, 513, 4, 0.6, 0, 0),      # G = 7, 2-tier fp16 + int8
    (3, 4, 1, 256, 77, 4, 0.7, 1, 0),        # d = 256, fp16 + int8
    (2, 16, 1, 64, 300, 0, 0.25, 1, 0),      # G = 16, all int4
    (2, 8, 4, 128, 1000, 4, 0.3, 0, 1),      # dropped tokens
    (1, 2, 2, 64, 1, 0, 1.0, 1, 0),          # one token
    # the matrix-core body: 4x4x4 p.V for G <= 4, 16x16x32 above
    (2, 16, 2, 256, 700, 4, 0.3, 1, 0),      # d = 256, G = 8: int8 + int4
    (1, 16, 1, 128, 600, 4, 0.45, 1, 0),     # d = 128, G = 16 (the largest group)
    (2, 4, 4, 128, 333, 4, 0.5, 1, 0),       # d = 128, G = 1
    (1, 6, 2, 256, 200, 4, 0.4, 1, 0),       # d = 256, G = 3 (4x4x4 with a spare column)
    # enough chunks x layers (>= 512) for the one-wavefront-per-KV-head workgroups at d = 128
    (16, 32, 8, 128, 2048, 4, 0.5, 1, 0),    # G = 4, int8 tier: 32 chunks x 16 layers
    (16, 28, 4, 128, 2600, 4, 0.6, 0, 0),    # G = 7, 2-tier: int8 tier 33 chunks x 16 layers
    # d = 256 with 32 KV heads: the widest token span the buffer-addressed
    # tiles cover in these tests (2 x 32 rows a token), ragged last tile
    (1, 32, 32, 256, 333, 4, 0.3, 1, 0),
]


def _run(L, Hq, H, d, n, S, b, three, overflow, layers, seed=0, kv=make_kv):
    shape = sk.Shape(L, Hq, H, d)
    pl = sk.plan_make(shape, sk.Policy(n, S, three, b, overflow))
    opl = OP.make_plan(L, Hq, H, d, n, S, b, three, overflow)
    K, V = kv(500 + n, L, n, H, d)
    # keep the reconstruction finite: the edge rows reach the fp16 maximum
    K = np.clip(K.astype(np.float32), -1e3, 1e3).astype(np.float16)
    V = np.clip(V.astype(np.float32), -1e3, 1e3).astype(np.float16)
    _, _, amap, _ = OA.assign(tied_scores(seed + n, n), opl.n16, opl.n8, opl.n4, opl.sinks)
    payload_h = OQ.pack(K, V, amap, opl)
    buf = torch.empty(max(pl.payload_bytes, 1), dtype=torch.uint8, device="cuda")
    payload = buf[:pl.payload_bytes]
    payload.copy_(torch.from_numpy(payload_h))
    rng = np.random.default_rng(seed + 1)
    layer0, nl = layers
    q = (rng.standard_normal((nl, Hq, d)) * 0.5).astype(np.float16)
    qd = to_dev(q)
    out = Guarded(4 * nl * Hq * d)
    lse = Guarded(4 * nl * Hq)
    o_t = out.as_(torch.float32, (nl, Hq, d))
    l_t = lse.as_(torch.float32, (nl, Hq))
    sk.decode_attention(shape, pl, payload, qd, o_t, l_t, layer0=layer0)
    torch.cuda.synchronize()
    out.check()
    lse.check()
    lrange = range(layer0, layer0 + nl)
    want_o, want_lse = OD.attention(payload_h, amap, opl, lrange, H, d, q)
    vmax = _vmax(payload_h, amap, opl, lrange, H, d, Hq)
    return o_t.cpu().numpy(), l_t.cpu().numpy(), want_o, want_lse, vmax


@pytest.mark.parametrize("case", CASES, ids=lambda c: "L%d_Hq%d_H%d_d%d_n%d_S%d_b%s_t%d_o%d" % c)
def test_decode_attention(case):
    say("decode", case)
    L = case[0]
    o, lse, wo, wl, vmax = _run(*case, layers=(0, L))
    _check(o, lse, wo, wl, vmax, str(case))
    if L > 1:
        o, lse, wo, wl, vmax = _run(*case, layers=(L - 1, 1))
        _check(o, lse, wo, wl, vmax, str(case) + " last layer")


def test_decode_attention_at_layer_limit():
    """All 65,535 layers a shape admits in one call (the layer is the third
    dimension of the tier grids and the second of the merge's): fp16 sinks,
    int8 and int4 tokens of an 11-token request."""
    case = (65535, 4, 2, 64, 11, 2, 0.55, 1, 0)
    say("decode at the layer limit", case)
    o, lse, wo, wl, vmax = _run(*case, layers=(0, case[0]), kv=make_kv_deep)
    _check(o, lse, wo, wl, vmax, str(case))


def test_decode_nothing_sent():
    """Every token dropped (2-tier, budget only pays the sinks): o = 0, lse = -inf."""
    L, Hq, H, d, n = 1, 4, 2, 64, 40
    shape = sk.Shape(L, Hq, H, d)
    pl = sk.plan_make(shape, sk.Policy(n, 0, 0, 0.0, sk.OVERFLOW_DROP))
    assert pl.n_drop == n and pl.payload_bytes == 0
    payload = torch.empty(1, dtype=torch.uint8, device="cuda")[:0]
    q = torch.ones((1, Hq, d), dtype=torch.float16, device="cuda")
    o = torch.full((1, Hq, d), 7.0, dtype=torch.float32, device="cuda")
    lse = torch.zeros((1, Hq), dtype=torch.float32, device="cuda")
    sk.decode_attention(shape, pl, payload, q, o, lse)
    torch.cuda.synchronize()
    assert torch.count_nonzero(o) == 0
    assert bool(torch.isneginf(lse).all())


def test_decode_full_size_sampled_layers():
    """Mistral-7B shape at full length, all 32 layers in one call (the launch
    configuration the benchmark times); sampled layers against the oracle."""
    cfg = get_config("mistral7b")
    L, Hq, H, d, n = cfg.layers, cfg.q_heads, cfg.kv_heads, cfg.head_dim, cfg.tokens
    say("full-size decode", n)
    shape = sk.Shape(L, Hq, H, d)
    pol = sk.Policy(n, cfg.sinks, cfg.three_tier, cfg.budget)
    pl = sk.plan_make(shape, pol)
    opl = OP.make_plan(L, Hq, H, d, n, cfg.sinks, cfg.budget, cfg.three_tier)
    _, _, amap, _ = OA.assign(tied_scores(3, n), opl.n16, opl.n8, opl.n4, opl.sinks)
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
    md = to_dev(amap.view(np.int32))
    payload = torch.empty(pl.payload_bytes, dtype=torch.uint8, device="cuda")
    sk.pack(shape, pl, Kd, Vd, md, None, payload)
    rng = np.random.default_rng(9)
    q = (rng.standard_normal((L, Hq, d)) * 0.5).astype(np.float16)
    o = torch.empty((L, Hq, d), dtype=torch.float32, device="cuda")
    lse = torch.empty((L, Hq), dtype=torch.float32, device="cuda")
    sk.decode_attention(shape, pl, payload, to_dev(q), o, lse)
    torch.cuda.synchronize()
    og, lg = o.cpu().numpy(), lse.cpu().numpy()
    for layer in layers:
        # the oracle's payload bytes of this layer, from the host tensors
        one = OP.make_plan(1, Hq, H, d, n, cfg.sinks, cfg.budget, cfg.three_tier)
        ph = OQ.pack(hk[layer][None], hv[layer][None], amap, one)
        wo, wl = OD.layer_attention(ph, amap, one, 0, H, d, q[layer])
        vmax = _vmax(ph, amap, one, [0], H, d, Hq)
        _check(og[layer][None], lg[layer][None], wo[None], wl[None], vmax, f"layer {layer}")


@pytest.mark.parametrize("n,H,b", [(1000, 2, 0.35), (65536, 8, 0.45)])
def test_decode_needle_at_boundaries(n, H, b):
    """One token whose key points along q dominates the softmax (weight
    ~1 - 1e-6), so o must equal its v_hat row.  Moved to the first and last
    slot of every tier, to both sides of 64-token tile boundaries and of the
    chunk boundaries of the long request (128 tokens per chunk there), it
    shows that those positions are read, with the right value, by the
    wavefront that owns them."""
    L, d, S = 1, 128, 4
    Hq = 2 * H
    shape = sk.Shape(L, Hq, H, d)
    pl = sk.plan_make(shape, sk.Policy(n, S, 1, b))
    opl = OP.make_plan(L, Hq, H, d, n, S, b, 1)
    assert pl.n8 > 256 and pl.n4 > 256
    rng = np.random.default_rng(17)
    K = rng.standard_normal((L, n, H, d)).astype(np.float16)
    V = rng.standard_normal((L, n, H, d)).astype(np.float16)
    _, _, amap, _ = OA.assign(tied_scores(77, n), opl.n16, opl.n8, opl.n4, opl.sinks)
    tier, slot = amap >> 30, amap & 0x3FFFFFFF
    sign = np.where(rng.random(d) < 0.5, -1.0, 1.0)
    q = np.tile((0.5 * sign).astype(np.float16), (1, Hq, 1))
    md = to_dev(amap.view(np.int32))
    picks = []
    for t, N in enumerate((opl.n16, opl.n8, opl.n4)):
        for sl in sorted({0, N - 1, 63, 64, 127, 128, 255, 256, N // 2} & set(range(N))):
            picks.append(int(np.nonzero((tier == t) & (slot == sl))[0][0]))
    say("needle tokens", n, picks)
    payload = torch.empty(pl.payload_bytes, dtype=torch.uint8, device="cuda")
    o = torch.empty((1, Hq, d), dtype=torch.float32, device="cuda")
    Vd = to_dev(V)
    for j in picks:
        Kn = K.copy()
        Kn[0, j] = (4.0 * sign).astype(np.float16)          # exact in every tier
        sk.pack(shape, pl, to_dev(Kn), Vd, md, None, payload)
        sk.decode_attention(shape, pl, payload, to_dev(q), o)
        torch.cuda.synchronize()
        got = o.cpu().numpy()[0]
        # v_hat of token j alone: its row through the pack oracle's quantizer
        t = int(tier[j])
        for h in range(Hq):
            g = h // (Hq // H)
            row = V[0, j, g][None].astype(np.float16)
            if t == 0:
                want = row[0].astype(np.float64)
            else:
                codes, s16 = OQ.quantize_rows(row, OQ.QMAX[t])
                want = OQ.dequantize_rows(codes, s16)[0].astype(np.float64)
            err = np.abs(got[h] - want).max()
            assert err <= 1e-3 * np.abs(want).max(), (j, t, int(slot[j]), h, err)


@pytest.mark.parametrize("name", ["qwen25_7b_2tier", "gemma2_9b"])
def test_decode_full_size_other_shapes(name):
    """The Qwen2.5-7B-shaped 2-tier request (query groups of 7 heads) and the
    Gemma-2-9B-shaped one (d = 256, b = 0.3: mostly int4) at full length, all
    layers in one call; sampled layers against the oracle."""
    cfg = get_config(name)
    L, Hq, H, d, n = cfg.layers, cfg.q_heads, cfg.kv_heads, cfg.head_dim, cfg.tokens
    say("full-size decode", name, n)
    shape = sk.Shape(L, Hq, H, d)
    pl = sk.plan_make(shape, sk.Policy(n, cfg.sinks, cfg.three_tier, cfg.budget))
    opl = OP.make_plan(L, Hq, H, d, n, cfg.sinks, cfg.budget, cfg.three_tier)
    _, _, amap, _ = OA.assign(tied_scores(4, n), opl.n16, opl.n8, opl.n4, opl.sinks)
    layers = sorted({1, L - 2})
    Kd = torch.empty((L, n, H, d), dtype=torch.float16, device="cuda")
    Vd = torch.empty_like(Kd)
    hk, hv = {}, {}
    for layer in range(L):
        k, v = gen.keys(cfg, layer), gen.values(cfg, layer)
        Kd[layer].copy_(torch.from_numpy(k))
        Vd[layer].copy_(torch.from_numpy(v))
        if layer in layers:
            hk[layer], hv[layer] = k, v
    md = to_dev(amap.view(np.int32))
    payload = torch.empty(pl.payload_bytes, dtype=torch.uint8, device="cuda")
    sk.pack(shape, pl, Kd, Vd, md, None, payload)
    del Kd, Vd
    rng = np.random.default_rng(10)
    q = (rng.standard_normal((L, Hq, d)) * 0.5).astype(np.float16)
    o = torch.empty((L, Hq, d), dtype=torch.float32, device="cuda")
    lse = torch.empty((L, Hq), dtype=torch.float32, device="cuda")
    sk.decode_attention(shape, pl, payload, to_dev(q), o, lse)
    torch.cuda.synchronize()
    og, lg = o.cpu().numpy(), lse.cpu().numpy()
    one = OP.make_plan(1, Hq, H, d, n, cfg.sinks, cfg.budget, cfg.three_tier)
    for layer in layers:
        say("checking layer", layer)
        ph = OQ.pack(hk[layer][None], hv[layer][None], amap, one)
        wo, wl = OD.layer_attention(ph, amap, one, 0, H, d, q[layer])
        vmax = _vmax(ph, amap, one, [0], H, d, Hq)
        _check(og[layer][None], lg[layer][None], wo[None], wl[None], vmax, f"{name} layer {layer}")
