"""GPU parity of the score variants of Algorithm 1 "score tokens" (SpectrumKV
paper): the recency weighting of the §4.3 importance formula and the KV-norm
fallback, each against the float64 oracle.

Tolerances follow from the arithmetic the kernels document:
  - recency: double-precision product rounded once to fp32, so the result is
    within one fp32 ulp of the oracle's (2^-23 relative); below the smallest
    normal fp32 (2^-126) either rounding of a denormal is accepted; lambda = 0
    returns the input bit for bit.
  - KV-norm: fp32 sums in a fixed order, relative error at most
    (m + 16) * 2^-24 with m = ceil(L * ceil(H * d / 512) / 8)."""

import math

import numpy as np
import pytest
import torch

from oracle import assign as OA
from oracle import plan as OP
from oracle import score as OS
import serving_sk_score_amd as sk
from workloads import gen, get_config
from tests.gpu_helpers import Guarded, make_kv, say, tied_scores, to_dev, u32

pytestmark = pytest.mark.gpu

TINY = 2.0 ** -126


def _recency_check(got, want):
    err = np.abs(got.astype(np.float64) - want.astype(np.float64))
    bound = 2.0 ** -23 * np.abs(want.astype(np.float64)) + TINY
    worst = int(np.argmax(err - bound))
    assert np.all(err <= bound), f"recency: err {err[worst]:.3g} > {bound[worst]:.3g} at {worst}"


@pytest.mark.parametrize("n", [1, 2, 255, 65536])
@pytest.mark.parametrize("lam", [0.0, 1e-4, 0.02, 0.7, 40.0])
def test_recency_weight(n, lam):
    say("recency", n, lam)
    s = tied_scores(100 + n, n)
    s_in = to_dev(s)
    out = Guarded(4 * n)
    sk.recency_weight(s_in, lam, out.as_(torch.float32, (n,)))
    torch.cuda.synchronize()
    out.check()
    got = out.as_(torch.float32, (n,)).cpu().numpy()
    want = OS.to_fp32(OS.recency_weight(s.astype(np.float64), lam))
    if lam == 0.0:
        assert np.array_equal(got.view(np.uint32), s.view(np.uint32))
    _recency_check(got, want)
    # in place gives the same bits
    sk.recency_weight(s_in, lam, s_in)
    torch.cuda.synchronize()
    assert np.array_equal(s_in.cpu().numpy().view(np.uint32), got.view(np.uint32))


def test_recency_rejects_bad_lambda_and_overlap():
    s = torch.ones(16, dtype=torch.float32, device="cuda")
    for lam in (-1e-3, math.inf, math.nan):
        with pytest.raises(sk.SkError):
            sk.recency_weight(s, lam)
    big = torch.ones(32, dtype=torch.float32, device="cuda")
    with pytest.raises(sk.SkError):
        sk.recency_weight(big[:16], 0.1, big[8:24])     # partial overlap
    e = torch.empty(0, dtype=torch.float32, device="cuda")
    sk.recency_weight(e, 0.5, e)                        # empty request


def _kvnorm_rtol(L, H, d):
    m = math.ceil(L * math.ceil(H * d / 512) / 8)
    return (m + 16) * 2.0 ** -24


def _kvnorm_check(got, want, rtol, tag):
    got = got.astype(np.float64)
    zero = want == 0
    assert np.all(got[zero] == 0), f"{tag}: zero keys gave a non-zero score"
    rel = np.abs(got[~zero] - want[~zero]) / want[~zero]
    if rel.size:
        worst = int(np.argmax(rel))
        assert rel.max() <= rtol, f"{tag}: rel err {rel.max():.3g} > {rtol:.3g} at {worst}"


KV_CASES = [
    # L, H, d, n
    (1, 2, 64, 256),     # tiny shape: one partial batch, 16 of 64 lanes live
    (3, 3, 128, 1000),   # 48 pieces per layer
    (2, 8, 128, 77),     # two wave steps per layer
    (5, 1, 256, 33),     # single KV head, d = 256
    (7, 12, 64, 99),     # second wave step of each layer half live, last batch partial
    (42, 8, 256, 300),   # Gemma-2-9B heads: 21 whole batches
    (32, 8, 128, 1025),  # Mistral-7B heads, ragged n
]


@pytest.mark.parametrize("case", KV_CASES, ids=lambda c: "L%d_H%d_d%d_n%d" % c)
def test_kvnorm(case):
    L, H, d, n = case
    say("kvnorm", case)
    K, _ = make_kv(300 + n, L, n, H, d)
    K[:, n // 2] = 0                                   # a token with all-zero keys
    shape = sk.Shape(L, H, H, d)
    out = Guarded(4 * n)
    score = out.as_(torch.float32, (n,))
    Kd = to_dev(K)
    sk.score_kvnorm(shape, Kd, score)
    torch.cuda.synchronize()
    out.check()
    got = score.cpu().numpy()
    _kvnorm_check(got, OS.kv_norm_score(K), _kvnorm_rtol(L, H, d), str(case))
    # accumulate: the second call adds the same values, exactly doubling them
    sk.score_kvnorm(shape, Kd, score, accumulate=True)
    torch.cuda.synchronize()
    out.check()
    assert np.array_equal(score.cpu().numpy(), got * np.float32(2))


def test_kvnorm_per_layer_accumulation_matches_whole():
    """Calling once per layer (n_layers = 1, accumulating) matches the oracle
    with the same bound as one call over all layers."""
    L, H, d, n = 4, 2, 128, 130
    K, _ = make_kv(7, L, n, H, d)
    out = torch.empty(n, dtype=torch.float32, device="cuda")
    for layer in range(L):
        sk.score_kvnorm(sk.Shape(1, H, H, d), to_dev(K[layer:layer + 1]), out,
                        accumulate=layer > 0)
    torch.cuda.synchronize()
    _kvnorm_check(out.cpu().numpy(), OS.kv_norm_score(K), _kvnorm_rtol(L, H, d) + L * 2.0 ** -24,
                  "per-layer")


def test_kvnorm_fallback_drives_assignment():
    """The fallback score feeds tier assignment: the GPU map equals the
    oracle's assignment of the GPU's own fp32 scores."""
    cfg = get_config("tiny")
    L, Hq, H, d, n = cfg.layers, cfg.q_heads, cfg.kv_heads, cfg.head_dim, cfg.tokens
    K = np.stack([gen.keys(cfg, layer) for layer in range(L)])
    shape = sk.Shape(L, Hq, H, d)
    score = torch.empty(n, dtype=torch.float32, device="cuda")
    sk.score_kvnorm(shape, to_dev(K), score)
    pol = sk.Policy(n, cfg.sinks, cfg.three_tier, cfg.budget)
    pl = sk.plan_make(shape, pol)
    amap = torch.empty(n, dtype=torch.int32, device="cuda")
    order = torch.empty(n, dtype=torch.int32, device="cuda")
    sk.assign_tiers(pol, pl, score, amap, order)
    torch.cuda.synchronize()
    sg = score.cpu().numpy()
    _kvnorm_check(sg, OS.kv_norm_score(K), _kvnorm_rtol(L, H, d), "tiny")
    opl = OP.make_plan(L, Hq, H, d, n, cfg.sinks, cfg.budget, cfg.three_tier)
    _, _, want_map, want_order = OA.assign(sg, opl.n16, opl.n8, opl.n4, opl.sinks)
    assert np.array_equal(u32(amap), want_map)
    assert np.array_equal(u32(order), want_order)


def test_kvnorm_full_size_sampled():
    """Mistral-7B shape at full length (the launch configuration the benchmark
    times); the oracle checks sampled tokens, which are independent."""
    cfg = get_config("mistral7b")
    L, Hq, H, d, n = cfg.layers, cfg.q_heads, cfg.kv_heads, cfg.head_dim, cfg.tokens
    rng = np.random.default_rng(5)
    cols = np.unique(np.concatenate([np.arange(8), np.arange(n - 8, n),
                                     rng.integers(0, n, 48)]))
    say("full-size kvnorm", n, "sampled", cols.size)
    Kd = torch.empty((L, n, H, d), dtype=torch.float16, device="cuda")
    Ks = np.empty((L, cols.size, H, d), dtype=np.float16)
    for layer in range(L):
        k = gen.keys(cfg, layer)
        Kd[layer].copy_(torch.from_numpy(k))
        Ks[layer] = k[cols]
    score = torch.empty(n, dtype=torch.float32, device="cuda")
    sk.score_kvnorm(sk.Shape(L, Hq, H, d), Kd, score)
    torch.cuda.synchronize()
    got = score.cpu().numpy()
    assert np.all(np.isfinite(got)) and np.all(got > 0)
    _kvnorm_check(got[cols], OS.kv_norm_score(Ks), _kvnorm_rtol(L, H, d), "mistral7b")
