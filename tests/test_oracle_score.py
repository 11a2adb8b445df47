"""Pins of the oracle's importance score (causal softmax column sums).

What fixes the expected values: invariants of a row-stochastic causal
softmax, closed forms (n = 1, equal keys -> harmonic numbers, a designed
two-token case with logits chosen by hand), brute force with scalar
``math.exp`` on tiny inputs, and torch's float64 softmax as a library routine.
"""

import math

import numpy as np
import pytest
import torch

from oracle import score as SC
from workloads import get_config, gen


def _rand(n, Hq, Hkv, d, seed, scale=1.0):
    r = np.random.default_rng(seed)
    q = (r.standard_normal((n, Hq, d)) * scale).astype(np.float16)
    k = (r.standard_normal((n, Hkv, d)) * scale).astype(np.float16)
    return q, k


def test_single_token():
    q, k = _rand(1, 4, 2, 64, 0)
    assert SC.layer_score(q, k)[0] == pytest.approx(4.0, rel=1e-15)


def test_row_stochastic_sum_and_first_token():
    cfg = get_config("tiny")
    q = gen.queries(cfg, 0)
    k = gen.keys(cfg, 0)
    a = SC.layer_score(q, k)
    n, Hq = q.shape[0], q.shape[1]
    assert a.sum() == pytest.approx(Hq * n, rel=1e-12)   # every row sums to 1
    assert a[0] >= Hq - 1e-12                            # p_00 = 1 in every head
    assert np.all(a > 0)


def _harmonic(m):
    return sum(1.0 / t for t in range(1, m + 1))


def test_equal_keys_harmonic():
    # all keys equal -> p_ij = 1/(i+1) -> A_j = H * (H_n - H_j)
    n, Hq, Hkv, d = 40, 4, 2, 64
    q, _ = _rand(n, Hq, Hkv, d, 1)
    k = np.tile(np.random.default_rng(2).standard_normal((1, Hkv, d)).astype(np.float16), (n, 1, 1))
    a = SC.layer_score(q, k)
    want = np.array([Hq * (_harmonic(n) - _harmonic(j)) for j in range(n)])
    np.testing.assert_allclose(a, want, rtol=1e-12)


def test_zero_queries_harmonic():
    n, Hq, Hkv, d = 33, 2, 1, 128
    _, k = _rand(n, Hq, Hkv, d, 3)
    q = np.zeros((n, Hq, d), dtype=np.float16)
    a = SC.layer_score(q, k)
    want = np.array([Hq * (_harmonic(n) - _harmonic(j)) for j in range(n)])
    np.testing.assert_allclose(a, want, rtol=1e-12)


@pytest.mark.parametrize("d", [64, 128, 256])
def test_two_token_closed_form(d):
    # One head.  q_1 . (k_0 - k_1) = sqrt(d) * ln 3 would make p_10 = 3/4, but
    # fp16 inputs cannot hit ln 3 exactly, so choose integer logit gaps:
    # q_1 = c e_0, k_0 = e_0, k_1 = 0  ->  s_10 = c / sqrt(d), s_11 = 0,
    # p_10 = 1 / (1 + exp(-c / sqrt(d))).  A_0 = 1 + p_10, A_1 = 1 - p_10.
    c = 2.0
    q = np.zeros((2, 1, d), dtype=np.float16)
    k = np.zeros((2, 1, d), dtype=np.float16)
    q[1, 0, 0] = c
    q[0, 0, 5] = 3.0            # query 0 sees only key 0: p_00 = 1 whatever it is
    k[0, 0, 0] = 1.0
    p10 = 1.0 / (1.0 + math.exp(-c / math.sqrt(d)))
    a = SC.layer_score(q, k)
    np.testing.assert_allclose(a, [1.0 + p10, 1.0 - p10], rtol=1e-14)


def test_gqa_contiguous_groups():
    # H_q = 4, H_kv = 2: heads 0,1 read KV head 0 and heads 2,3 read KV head 1.
    # KV head 0 has equal keys (harmonic); KV head 1 has k_1 = 0, k_0 = e_0.
    # Heads 0,1 query 4 e_0 and heads 2,3 query 8 e_0 -> per-head two-token
    # closed form on n = 2.
    d = 64
    q = np.zeros((2, 4, d), dtype=np.float16)
    k = np.zeros((2, 2, d), dtype=np.float16)
    q[:, 0:2, 0] = 4.0
    q[:, 2:4, 0] = 8.0
    k[:, 0, 1] = 1.0                      # group 0: identical keys
    k[0, 1, 0] = 1.0                      # group 1: k_0 = e_0, k_1 = 0
    p10 = 1.0 / (1.0 + math.exp(-8.0 / 8.0))
    want = 2 * np.array([1.5, 0.5]) + 2 * np.array([1 + p10, 1 - p10])
    np.testing.assert_allclose(SC.layer_score(q, k), want, rtol=1e-14)
    # the interleaved mapping (h % H_kv) would give a different answer
    alt = np.zeros(2)
    for h in range(4):
        alt += SC.head_column_sums(q[:, h, :], k[:, h % 2, :])
    assert not np.allclose(alt, want)


def _brute(q, k):
    n, Hq, d = q.shape
    Hkv = k.shape[1]
    out = [0.0] * n
    for h in range(Hq):
        g = h // (Hq // Hkv)
        for i in range(n):
            s = []
            for j in range(i + 1):
                s.append(sum(float(q[i, h, t]) * float(k[j, g, t]) for t in range(d)) / math.sqrt(d))
            m = max(s)
            e = [math.exp(x - m) for x in s]
            z = sum(e)
            for j in range(i + 1):
                out[j] += e[j] / z
    return np.array(out)


@pytest.mark.parametrize("n,Hq,Hkv,d,scale", [(5, 2, 1, 64, 1.0), (12, 4, 2, 64, 2.0), (9, 3, 3, 128, 0.5)])
def test_brute_force(n, Hq, Hkv, d, scale):
    q, k = _rand(n, Hq, Hkv, d, n, scale)
    np.testing.assert_allclose(SC.layer_score(q, k), _brute(q, k), rtol=1e-12)


def test_torch_softmax_library():
    n, Hq, Hkv, d = 300, 4, 2, 64
    q, k = _rand(n, Hq, Hkv, d, 7, 1.5)
    want = torch.zeros(n, dtype=torch.float64)
    mask = torch.ones(n, n, dtype=torch.bool).tril()
    for h in range(Hq):
        g = h // (Hq // Hkv)
        s = torch.from_numpy(q[:, h, :].astype(np.float64)) @ torch.from_numpy(k[:, g, :].astype(np.float64)).T
        s = s / math.sqrt(d)
        s = s.masked_fill(~mask, float("-inf"))
        want += torch.softmax(s, dim=1).sum(0)
    np.testing.assert_allclose(SC.layer_score(q, k), want.numpy(), rtol=1e-12)
    lse = torch.logsumexp(
        (torch.from_numpy(q[:, 1, :].astype(np.float64)) @ torch.from_numpy(k[:, 0, :].astype(np.float64)).T
         / math.sqrt(d)).masked_fill(~mask, float("-inf")), dim=1)
    np.testing.assert_allclose(SC.head_row_lse(q[:, 1, :], k[:, 0, :]), lse.numpy(), rtol=1e-13)


def test_blocking_invariance_and_column_sample():
    # rows crossing the internal block size, and the sampled-column variant
    n, Hq, Hkv, d = 1100, 2, 1, 64
    q, k = _rand(n, Hq, Hkv, d, 11)
    full = SC.layer_score(q, k)
    old = SC._BLOCK
    try:
        SC._BLOCK = 97
        np.testing.assert_allclose(SC.layer_score(q, k), full, rtol=1e-12)
    finally:
        SC._BLOCK = old
    cols = [0, 5, 511, 512, 513, 1000, 1099]
    np.testing.assert_allclose(SC.layer_column_sample(q, k, cols), full[cols], rtol=1e-12)
    cols = [1050, 1090, 1099]
    np.testing.assert_allclose(SC.layer_column_sample(q, k, cols), full[cols], rtol=1e-12)


def test_fp32_rounding_is_nearest():
    x = np.array([1.0 + 2.0 ** -24, 1.0 + 3 * 2.0 ** -24, 0.1])
    f = SC.to_fp32(x)
    assert f.dtype == np.float32
    assert f[0] == np.float32(1.0)                      # tie -> even
    assert f[1] == np.float32(1.0 + 2.0 ** -22)         # tie -> even (up)
    assert abs(float(f[2]) - 0.1) <= 2.0 ** -28


# ---------------------------------------------------------------- variants --
# Recency weighting I_j = A_j exp(-lambda Delta_j) and the KV-norm fallback
# (Algorithm 1 "score tokens").  Pins: closed forms, brute force with scalar
# math on tiny inputs, exact scaling.

def test_recency_lambda_zero_is_identity():
    a = np.random.default_rng(1).random(37) * 10
    assert np.array_equal(SC.recency_weight(a, 0.0), a)


def test_recency_closed_form_on_constant_scores():
    n, lam = 50, 0.07
    w = SC.recency_weight(np.full(n, 3.0), lam)
    assert w[-1] == 3.0                                   # Delta = 0 for the last token
    assert w[0] == pytest.approx(3.0 * math.exp(-lam * (n - 1)), rel=1e-15)
    ratio = w[1:] / w[:-1]
    assert np.allclose(ratio, math.exp(lam), rtol=1e-14)  # geometric in the position
    assert np.all(np.diff(w) > 0)                         # recent tokens rank higher


def test_recency_brute_force():
    rng = np.random.default_rng(2)
    for n in (1, 2, 9):
        a = rng.random(n) * 5
        lam = float(rng.random())
        want = [a[j] * math.exp(-lam * (n - 1 - j)) for j in range(n)]
        assert np.allclose(SC.recency_weight(a, lam), want, rtol=1e-15, atol=0)


def test_kv_norm_constant_keys():
    L, n, H, d = 3, 5, 2, 64
    ks = np.full((L, n, H, d), -0.75, dtype=np.float16)
    want = L * H * 0.75 * math.sqrt(d)
    assert np.allclose(SC.kv_norm_score(ks), want, rtol=1e-14)


def test_kv_norm_brute_force_and_scaling():
    rng = np.random.default_rng(3)
    L, n, H, d = 2, 4, 3, 8
    ks = rng.standard_normal((L, n, H, d)).astype(np.float16)
    want = []
    for j in range(n):
        tot = 0.0
        for layer in range(L):
            for g in range(H):
                tot += math.sqrt(sum(float(x) ** 2 for x in ks[layer, j, g]))
        want.append(tot)
    got = SC.kv_norm_score(ks)
    assert np.allclose(got, want, rtol=1e-13)
    # doubling every key (exact in fp16 here) doubles every score exactly
    assert np.array_equal(SC.kv_norm_score(ks * np.float16(2)), 2 * got)
    # a key with a single non-zero element contributes its magnitude
    one = np.zeros((1, 1, 1, d), dtype=np.float16)
    one[0, 0, 0, 3] = -5.5
    assert SC.kv_norm_score(one)[0] == 5.5
