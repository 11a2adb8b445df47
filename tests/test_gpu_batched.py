"""The batched serving mix on the GPU: 16 Mistral-7B-shaped requests with
seeded log-uniform lengths in [1024, 65536], each scored, assigned to tiers,
packed at every budget of the sweep {0.3, 0.5, 0.7} (3-tier, S = 4) and
unpacked into one shared paged fp16 cache of 16-token blocks through a seeded
permutation of the block pool.

Every request runs at its full length on one sampled layer (layer r mod 32):
  - scores: positive, finite, and the row-stochastic invariant
    sum_j A_j = H_q * n for every request; against the fp64 oracle on the
    whole layer of the shortest request and on sampled late columns of the
    longest one;
  - tiers: the GPU map equals the oracle's assignment of the GPU's own fp32
    scores, bit for bit;
  - payload and paged cache: bit-exact against the oracle's quantizer and
    paged unpack, including the blocks of every other request staying
    untouched."""

import numpy as np
import pytest
import torch

from oracle import assign as OA
from oracle import plan as OP
from oracle import quant as OQ
from oracle import score as OS
import serving_sk_score_amd as sk
from workloads import gen, get_config
from tests.gpu_helpers import say, to_dev, u32

pytestmark = pytest.mark.gpu

RTOL = 2e-3
FILL = 0x4248   # fp16 3.140625: marks cache rows no request has written


def _close(got, want, tag):
    rel = np.abs(got - want) / np.abs(want)
    worst = int(np.argmax(rel))
    assert rel.max() <= RTOL, f"{tag}: max rel err {rel.max():.3g} at {worst}"


def test_batched_mix_paged():
    cfg = get_config("batched_mix")
    Hq, H, d, bs = cfg.q_heads, cfg.kv_heads, cfg.head_dim, cfg.block_size
    lengths = gen.request_lengths(cfg)
    tables, num_blocks = gen.block_tables(cfg, lengths)
    say("batched mix lengths", lengths, "blocks", num_blocks)
    assert len(lengths) == cfg.requests
    assert all(cfg.len_lo <= n <= cfg.len_hi for n in lengths)
    shape1 = sk.Shape(1, Hq, H, d)
    cshape = (1, num_blocks, bs, H, d)
    kc = torch.full(cshape, 0, dtype=torch.int16, device="cuda").fill_(FILL).view(torch.float16)
    vc = torch.full(cshape, 0, dtype=torch.int16, device="cuda").fill_(FILL).view(torch.float16)
    kcw = np.full(cshape, FILL, dtype=np.int16).view(np.float16)
    vcw = np.full(cshape, FILL, dtype=np.int16).view(np.float16)
    shortest = int(np.argmin(lengths))
    longest = int(np.argmax(lengths))
    for r, n in enumerate(lengths):
        layer = r % cfg.layers
        say(f"request {r}: n={n} layer={layer}")
        k = gen.keys(cfg, layer, n, request=r)
        v = gen.values(cfg, layer, n, request=r)
        q = gen.queries(cfg, layer, n, request=r, k=k)
        kd, vd = to_dev(k[None]), to_dev(v[None])
        score = torch.empty(n, dtype=torch.float32, device="cuda")
        sk.score(shape1, to_dev(q), kd[0], score, False)
        torch.cuda.synchronize()
        sg = score.cpu().numpy()
        assert np.all(np.isfinite(sg)) and np.all(sg > 0)
        assert abs(sg.astype(np.float64).sum() - Hq * n) <= 1e-4 * Hq * n
        if r == shortest:
            say("oracle layer score", n)
            _close(sg.astype(np.float64), OS.layer_score(q, k), f"request {r}")
        if r == longest:
            cols = np.arange(n - 24, n)
            say("oracle sampled columns", n)
            _close(sg[cols].astype(np.float64), OS.layer_column_sample(q, k, cols), f"request {r}")
        bt = tables[r]
        for b in cfg.budgets:
            pl = sk.plan_make(shape1, sk.Policy(n, cfg.sinks, cfg.three_tier, b))
            opl = OP.make_plan(1, Hq, H, d, n, cfg.sinks, b, cfg.three_tier)
            assert pl.counts() == (opl.n16, opl.n8, opl.n4)
            amap = torch.empty(n, dtype=torch.int32, device="cuda")
            order = torch.empty(n, dtype=torch.int32, device="cuda")
            sk.assign_tiers(sk.Policy(n, cfg.sinks, cfg.three_tier, b), pl, score, amap, order)
            payload = torch.empty(pl.payload_bytes, dtype=torch.uint8, device="cuda")
            sk.pack(shape1, pl, kd, vd, amap, order, payload)
            sk.unpack_paged(shape1, pl, payload, amap, kc, vc, to_dev(bt), bs)
            torch.cuda.synchronize()
            gmap = u32(amap)
            _, _, want_map, want_order = OA.assign(sg, opl.n16, opl.n8, opl.n4, opl.sinks)
            assert np.array_equal(gmap, want_map), (r, b)
            assert np.array_equal(u32(order), want_order), (r, b)
            want = OQ.pack(k[None], v[None], gmap, opl)
            assert np.array_equal(payload.cpu().numpy(), want), (r, b)
            OQ.unpack_paged(want, gmap, opl, 1, H, d, bt, kcw, vcw, bs)
            blocks = torch.from_numpy(bt.astype(np.int64)).cuda()
            assert np.array_equal(kc[0, blocks].cpu().numpy().view(np.int16),
                                  kcw[0, bt].view(np.int16)), (r, b)
            assert np.array_equal(vc[0, blocks].cpu().numpy().view(np.int16),
                                  vcw[0, bt].view(np.int16)), (r, b)
    # every block was written by exactly its request; nothing else changed
    say("whole cache compare")
    assert np.array_equal(kc.cpu().numpy().view(np.int16), kcw.view(np.int16))
    assert np.array_equal(vc.cpu().numpy().view(np.int16), vcw.view(np.int16))
