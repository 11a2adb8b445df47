"""Pins of the oracle's quantizer, payload and unpack.

What fixes the expected values: hand-worked rows (``tests/golden``), the
properties of symmetric absmax quantization (code ranges, the absmax element
hitting +-qmax, the half-step error bound), the uniform int8 / int4 special
cases (b = 0.5 / 0.25 with no sinks, SpectrumKV paper §7.5) against a few
lines of torch on the CPU, the fp16 tier being the identity, the payload size
closed form, and dense == gather(paged).
"""

import os

import numpy as np
import pytest
import torch

from oracle import assign as A
from oracle import plan as P
from oracle import quant as Q

GOLD = os.path.join(os.path.dirname(__file__), "golden", "quant_examples.txt")


def _golden():
    out = []
    for line in open(GOLD):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        f = [x.strip() for x in line.split("|")]
        out.append(dict(name=f[0], qmax=int(f[1]),
                        x=[float(v) for v in f[2].split()],
                        scale=float(f[3]),
                        codes=[int(v) for v in f[4].split()],
                        packed=bytes.fromhex(f[5].replace(" ", "")),
                        deq=[float(v) for v in f[6].split()]))
    return out


@pytest.mark.parametrize("case", _golden(), ids=lambda c: c["name"])
def test_golden_rows(case):
    x = np.array(case["x"], dtype=np.float64)
    x16 = x.astype(np.float16)
    assert np.array_equal(x16.astype(np.float64), x), "golden inputs must be exact fp16"
    codes, s16 = Q.quantize_rows(x16[None, :], case["qmax"])
    assert float(s16[0]) == case["scale"]
    assert codes[0].tolist() == case["codes"]
    enc = codes[0].view(np.uint8) if case["qmax"] == 127 else Q.encode_int4(codes[0])
    assert bytes(enc.tobytes()) == case["packed"]
    deq = Q.dequantize_rows(codes, s16)[0].astype(np.float64)
    assert deq.tolist() == case["deq"]


def test_int4_nibbles_bijective():
    vals = np.arange(-7, 8, dtype=np.int8)
    grid = np.array(np.meshgrid(vals, vals)).reshape(2, -1).T.copy()   # all pairs
    packed = Q.encode_int4(grid)
    assert np.array_equal(Q.decode_int4(packed), grid)
    assert len(set(packed[:, 0].tolist())) == 225


@pytest.mark.parametrize("qmax", [127, 7])
def test_quantizer_properties(qmax):
    r = np.random.default_rng(qmax)
    x = (r.standard_normal((4000, 128)) * np.exp(r.uniform(-12, 6, (4000, 1)))).astype(np.float16)
    x[0] = 0
    codes, s16 = Q.quantize_rows(x, qmax)
    assert codes.min() >= -qmax and codes.max() <= qmax
    s = s16.astype(np.float64)
    a = np.abs(x.astype(np.float64)).max(axis=1)
    normal = s >= 2.0 ** -14
    assert np.all(np.abs(codes[normal]).max(axis=1) == qmax)
    err = np.abs(x.astype(np.float64) - codes.astype(np.float64) * s[:, None])
    bound = 0.5 * s + np.maximum(0.0, a - qmax * s)
    assert np.all(err <= bound[:, None] * (1 + 1e-12) + 1e-30)
    deq = Q.dequantize_rows(codes, s16).astype(np.float64)
    assert np.all(np.abs(deq - codes * s[:, None]) <= np.abs(codes * s[:, None]) * 2.0 ** -11 + 2.0 ** -25)


def _textbook(x, qmax):
    # per-token symmetric absmax quantization written with torch on the CPU
    t = torch.from_numpy(x.astype(np.float32))
    scale = (t.abs().amax(dim=-1, keepdim=True) / qmax).half().float()
    q = torch.where(scale > 0, torch.round(t / torch.where(scale > 0, scale, torch.ones_like(scale))),
                    torch.zeros_like(t)).clamp(-qmax, qmax)
    return q.to(torch.int8).numpy(), scale.squeeze(-1).half().numpy()


@pytest.mark.parametrize("b,qmax", [(0.5, 127), (0.25, 7)])
def test_uniform_special_case(b, qmax):
    L, H, d, n = 2, 2, 64, 50
    r = np.random.default_rng(5)
    K = r.standard_normal((L, n, H, d)).astype(np.float16)
    V = (r.standard_normal((L, n, H, d)) * 3).astype(np.float16)
    pl = P.make_plan(L, H, H, d, n, 0, b, 1)
    tier_id = P.INT8 if qmax == 127 else P.INT4
    assert (pl.n16, pl.n8, pl.n4)[tier_id] == n
    _, _, amap, _ = A.assign(np.zeros(n, np.float32), pl.n16, pl.n8, pl.n4, 0)
    payload = Q.pack(K, V, amap, pl)
    assert payload.size == pl.payload_bytes
    rows = np.stack([K, V], axis=2)                  # [L][n][2][H][d], slot = token
    codes, s16 = _textbook(rows, qmax)
    if qmax == 127:
        got_codes = payload[pl.off_c8:pl.off_s8].view(np.int8).reshape(codes.shape)
        got_s = payload[pl.off_s8:pl.off_s4].view("<f2").reshape(s16.shape)
    else:
        got_codes = Q.decode_int4(payload[pl.off_c4:pl.off_s8].reshape(L, n, 2, H, d // 2))
        got_s = payload[pl.off_s4:].view("<f2").reshape(s16.shape)
    assert np.array_equal(got_codes, codes)
    assert np.array_equal(got_s.view(np.uint16), s16.view(np.uint16))


def test_fp16_tier_identity_and_roundtrip():
    L, Hq, H, d, n = 2, 4, 2, 128, 70
    r = np.random.default_rng(9)
    K = r.standard_normal((L, n, H, d)).astype(np.float16)
    V = r.standard_normal((L, n, H, d)).astype(np.float16)
    pl = P.make_plan(L, Hq, H, d, n, 4, 1.0, 1)
    _, _, amap, _ = A.assign(r.random(n).astype(np.float32), pl.n16, pl.n8, pl.n4, pl.sinks)
    Kh, Vh = Q.unpack_dense(Q.pack(K, V, amap, pl), amap, pl, L, H, d)
    assert np.array_equal(Kh.view(np.uint16), K.view(np.uint16))
    assert np.array_equal(Vh.view(np.uint16), V.view(np.uint16))


def test_mixed_roundtrip_and_paged():
    L, Hq, H, d, n, bs = 2, 4, 2, 64, 83, 16
    r = np.random.default_rng(10)
    K = r.standard_normal((L, n, H, d)).astype(np.float16)
    V = r.standard_normal((L, n, H, d)).astype(np.float16)
    pl = P.make_plan(L, Hq, H, d, n, 4, 0.45, 1)
    assert pl.n16 == 4 and pl.n8 > 0 and pl.n4 > 0
    tier, slot, amap, _ = A.assign(r.random(n).astype(np.float32), pl.n16, pl.n8, pl.n4, pl.sinks)
    payload = Q.pack(K, V, amap, pl)
    Kh, Vh = Q.unpack_dense(payload, amap, pl, L, H, d)
    for t, qmax in ((1, 127), (2, 7)):
        m = tier == t
        c, s = Q.quantize_rows(K[:, m], qmax)
        assert np.array_equal(Kh[:, m].view(np.uint16), Q.dequantize_rows(c, s).view(np.uint16))
    assert np.array_equal(Kh[:, tier == 0].view(np.uint16), K[:, tier == 0].view(np.uint16))
    # paged: scatter through a permuted block table, then gather back
    nb = (n + bs - 1) // bs
    total = nb + 3
    bt = r.permutation(total)[:nb].astype(np.int32)
    kc = np.full((L, total, bs, H, d), np.float16(7.0))
    vc = np.full((L, total, bs, H, d), np.float16(7.0))
    Q.unpack_paged(payload, amap, pl, L, H, d, bt, kc, vc, bs)
    j = np.arange(n)
    assert np.array_equal(kc[:, bt[j // bs], j % bs].view(np.uint16), Kh.view(np.uint16))
    assert np.array_equal(vc[:, bt[j // bs], j % bs].view(np.uint16), Vh.view(np.uint16))
    untouched = np.ones((total, bs), dtype=bool)
    untouched[bt[j // bs], j % bs] = False
    assert np.all(kc[:, untouched] == 7.0) and np.all(vc[:, untouched] == 7.0)


def test_int8_cosine_diagnostic():
    # qualitative match with the SpectrumKV paper's Table 8: int8 K/V cosine > 0.9999
    r = np.random.default_rng(3)
    x = r.standard_normal((2000, 128)).astype(np.float16)
    c, s = Q.quantize_rows(x, 127)
    y = Q.dequantize_rows(c, s).astype(np.float64)
    xx = x.astype(np.float64)
    cos = (xx * y).sum(1) / np.linalg.norm(xx, axis=1) / np.linalg.norm(y, axis=1)
    assert cos.mean() > 0.9999
