"""Pins of the decode-attention oracle (SpectrumKV §4.2; the Minima-KV page's
log-sum-exp merge): closed forms, torch's float64 scaled-dot-product
attention on the dequantized rows, exclusion of dropped tokens, token-order
independence and the merge identity."""

import math

import numpy as np
import torch

from oracle import assign as OA
from oracle import decode as OD
from oracle import plan as OP
from oracle import quant as OQ


def _setup(L, Hq, H, d, n, S, b, three, overflow=OP.REJECT, seed=0):
    rng = np.random.default_rng(seed)
    K = rng.standard_normal((L, n, H, d)).astype(np.float16)
    V = rng.standard_normal((L, n, H, d)).astype(np.float16)
    plan = OP.make_plan(L, Hq, H, d, n, S, b, three, overflow)
    sc = rng.random(n).astype(np.float32)
    _, _, amap, _ = OA.assign(sc, plan.n16, plan.n8, plan.n4, plan.sinks)
    payload = OQ.pack(K, V, amap, plan)
    q = rng.standard_normal((L, Hq, d)).astype(np.float16)
    return K, V, plan, amap, payload, q


def test_single_token_is_its_value():
    K, V, plan, amap, payload, q = _setup(1, 4, 2, 64, 1, 0, 1.0, 1)
    o, lse = OD.layer_attention(payload, amap, plan, 0, 2, 64, q[0])
    for h in range(4):
        g = h // 2
        assert np.array_equal(o[h], V[0, 0, g].astype(np.float64))
        want = float(K[0, 0, g].astype(np.float64) @ q[0, h].astype(np.float64)) / 8.0
        assert abs(lse[h] - want) < 1e-12


def test_equal_keys_average_the_values():
    L, Hq, H, d, n = 1, 2, 1, 64, 9
    K = np.tile(np.float16(0.5), (L, n, H, d))
    V = np.random.default_rng(1).standard_normal((L, n, H, d)).astype(np.float16)
    plan = OP.make_plan(L, Hq, H, d, n, 0, 1.0, 1)
    amap = np.arange(n, dtype=np.uint32)                     # all fp16, slot j
    payload = OQ.pack(K, V, amap, plan)
    q = np.random.default_rng(2).standard_normal((Hq, d)).astype(np.float16)
    o, lse = OD.layer_attention(payload, amap, plan, 0, H, d, q)
    assert np.allclose(o, V[0, :, 0].astype(np.float64).mean(axis=0), rtol=0, atol=1e-12)
    s = 0.5 * q.astype(np.float64).sum(axis=1) / 8.0
    assert np.allclose(lse, s + math.log(n), atol=1e-12)


def test_matches_torch_sdpa_on_the_dequantized_rows():
    L, Hq, H, d, n = 2, 8, 2, 128, 300
    K, V, plan, amap, payload, q = _setup(L, Hq, H, d, n, 4, 0.35, 1, seed=3)
    Kd, Vd = OQ.unpack_dense(payload, amap, plan, L, H, d)
    o, lse = OD.attention(payload, amap, plan, range(L), H, d, q)
    for layer in range(L):
        kt = torch.from_numpy(Kd[layer].astype(np.float64)).permute(1, 0, 2)   # [H][n][d]
        vt = torch.from_numpy(Vd[layer].astype(np.float64)).permute(1, 0, 2)
        kt = kt.repeat_interleave(Hq // H, dim=0)
        vt = vt.repeat_interleave(Hq // H, dim=0)
        qt = torch.from_numpy(q[layer].astype(np.float64))[:, None, :]         # [Hq][1][d]
        want = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt)[:, 0, :]
        assert np.allclose(o[layer], want.numpy(), rtol=1e-12, atol=1e-12)
        s = (qt @ kt.transpose(1, 2))[:, 0, :] / math.sqrt(d)
        assert np.allclose(lse[layer], torch.logsumexp(s, dim=1).numpy(), atol=1e-12)


def test_dropped_tokens_take_no_part():
    L, Hq, H, d, n = 1, 4, 2, 64, 200
    K, V, plan, amap, payload, q = _setup(L, Hq, H, d, n, 4, 0.3, 0, OP.DROP_OVERFLOW, seed=4)
    assert plan.n_drop > 0
    o, lse = OD.layer_attention(payload, amap, plan, 0, H, d, q[0])
    kept = np.nonzero((amap >> 30) <= 2)[0]
    Kd, Vd = OQ.unpack_dense(payload, amap, plan, L, H, d,
                             np.zeros((L, n, H, d), np.float16), np.zeros((L, n, H, d), np.float16))
    for h in range(Hq):
        g = h // 2
        s = Kd[0, kept, g].astype(np.float64) @ q[0, h].astype(np.float64) / 8.0
        w = np.exp(s - s.max())
        assert np.allclose(o[h], w @ Vd[0, kept, g].astype(np.float64) / w.sum(), atol=1e-12)


def test_merge_of_two_halves_is_the_whole():
    L, Hq, H, d, n = 1, 4, 2, 64, 120
    K, V, plan, amap, payload, q = _setup(L, Hq, H, d, n, 0, 1.0, 1, seed=5)
    o, lse = OD.layer_attention(payload, amap, plan, 0, H, d, q[0])
    parts = []
    for sel in (np.arange(n) < 50, np.arange(n) >= 50):
        # a request made of one half only: the other half is dropped
        m2 = amap.copy()
        m2[~sel] = np.uint32(3) << np.uint32(30)
        parts.append(OD.layer_attention(payload, m2, plan, 0, H, d, q[0]))
    om, lm = OD.merge(parts[0][0], parts[0][1], parts[1][0], parts[1][1])
    assert np.allclose(om, o, atol=1e-12) and np.allclose(lm, lse, atol=1e-12)


def test_nothing_sent():
    L, Hq, H, d, n = 1, 2, 1, 64, 10
    K, V, plan, amap, payload, q = _setup(L, Hq, H, d, n, 0, 1.0, 1, seed=6)
    none = np.full(n, np.uint32(3) << np.uint32(30), dtype=np.uint32)
    o, lse = OD.layer_attention(payload, none, plan, 0, H, d, q[0])
    assert np.all(o == 0) and np.all(np.isneginf(lse))
