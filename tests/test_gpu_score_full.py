"""Every column of the importance score at the longest lengths the workloads
have, against the fp64 oracle (SpectrumKV §4.3 "Importance scores",
Algorithm 1 "score tokens"): one KV group of a layer, so that all n
columns - the sink and early columns, whose sums run over tens of thousands
of query rows, as well as the late ones - are checked element by element at
the 2e-3 relative tolerance.

The score is additive over (layer, KV group) and the kernels compute each
group independently, so the group's query heads and its one KV head are
passed as a layer of their own (H_q = the group size, H_kv = 1).  That keeps
the grouping ratio, and with it the row pass's heads per workgroup and every
workgroup's work, exactly as in the full layer; the column sums are then the
oracle's layer score restricted to those heads.  The oracle runs one head
per thread (numpy releases the interpreter lock inside BLAS and ufuncs)."""

from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

from oracle import score as OS
import serving_sk_score_amd as sk
from workloads import gen, get_config
from tests.gpu_helpers import Guarded, say, to_dev

pytestmark = pytest.mark.gpu

RTOL = 2e-3


def _group_check(name, q, k, g, tag):
    n, Hq, d = q.shape
    R = Hq // k.shape[1]
    qg = np.ascontiguousarray(q[:, g * R:(g + 1) * R, :])
    kg = np.ascontiguousarray(k[:, g:g + 1, :])
    shape = sk.Shape(1, R, 1, d)
    out = Guarded(4 * n)
    say(f"{tag}: GPU score of KV group {g} ({R} heads), n={n}, d={d}")
    sk.score(shape, to_dev(qg), to_dev(kg), out.as_(torch.float32, (n,)), False)
    torch.cuda.synchronize()
    out.check()
    got = out.as_(torch.float32, (n,)).cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(got)) and np.all(got > 0)
    assert abs(got.sum() - R * n) <= 1e-4 * R * n, "row-stochastic invariant"
    say(f"{tag}: oracle (fp64), {R} heads on {R} threads ...")
    with ThreadPoolExecutor(R) as ex:
        parts = list(ex.map(lambda h: OS.head_column_sums(qg[:, h, :], kg[:, 0, :]), range(R)))
    want = np.sum(parts, axis=0)
    rel = np.abs(got - want) / want
    worst = int(np.argmax(rel))
    say(f"{tag}: max rel err {rel.max():.3g} at column {worst}; columns 0-63 max "
        f"{rel[:64].max():.3g}")
    assert rel.max() <= RTOL, (f"{tag}: column {worst}: {got[worst]} vs {want[worst]} "
                               f"(rel {rel[worst]:.3g})")


@pytest.mark.parametrize("name,layer,g", [("qwen25_7b_2tier", 0, 0), ("gemma2_9b", 0, 0)])
def test_every_column_one_group(name, layer, g):
    cfg = get_config(name)
    k = gen.keys(cfg, layer)
    q = gen.queries(cfg, layer, k=k)
    _group_check(name, q, k, g, f"{name} layer {layer}")


def test_every_column_longest_batched_request():
    """The 64,226-token request of the batched mix (Mistral-7B shape, 4 query
    heads per KV head), on the layer the batched test samples for it."""
    cfg = get_config("batched_mix")
    lengths = gen.request_lengths(cfg)
    r = int(np.argmax(lengths))
    n = lengths[r]
    layer = r % cfg.layers
    k = gen.keys(cfg, layer, n, request=r)
    q = gen.queries(cfg, layer, n, request=r, k=k)
    _group_check("batched_mix", q, k, 0, f"batched request {r} (n={n}) layer {layer}")


@pytest.mark.parametrize("name", ["mistral7b", "qwen25_7b_2tier", "gemma2_9b", "batched_mix"])
def test_all_layer_launch_full_size(name):
    """The launch configuration the benchmark times: every layer of a request
    at full size in one launch per pass (sk_score_rowlse_layers +
    sk_score_colsum_layers, and sk_score_layers), on the inputs the benchmark
    draws on the device.  The score must be bit for bit that of one sk_score
    call per layer, accumulating from the second layer on - the per-layer
    path the tests above and the per-layer full-size tests compare with the
    oracle - and meet the row-stochastic invariant sum_j A_j = L * H_q * n.
    For the batched mix, its longest request."""
    from workloads import gen_device as gd
    cfg = get_config(name)
    L, Hq, Hkv, d = cfg.layers, cfg.q_heads, cfg.kv_heads, cfg.head_dim
    if cfg.requests:
        lengths = gen.request_lengths(cfg)
        r = int(np.argmax(lengths))
        n = lengths[r]
    else:
        r, n = 0, cfg.tokens
    say("all-layer launch", name, dict(L=L, n=n, Hq=Hq, Hkv=Hkv, d=d))
    Q = torch.empty((L, n, Hq, d), dtype=torch.float16, device="cuda")
    K = torch.empty((L, n, Hkv, d), dtype=torch.float16, device="cuda")
    for layer in range(L):
        gd.keys(cfg, layer, n, r, out=K[layer])
        gd.queries(cfg, layer, n, r, k=K[layer], out=Q[layer])
    s1 = sk.Shape(1, Hq, Hkv, d)
    sL = sk.Shape(L, Hq, Hkv, d)
    want = torch.empty(n, dtype=torch.float32, device="cuda")
    for layer in range(L):
        sk.score(s1, Q[layer], K[layer], want, accumulate=layer > 0)
    lse = Guarded(4 * L * Hq * n)
    out = Guarded(4 * n)
    sk.score_rowlse_layers(sL, Q, K, lse.as_(torch.float32, (L, Hq, n)))
    sk.score_colsum_layers(sL, Q, K, lse.as_(torch.float32, (L, Hq, n)),
                           out.as_(torch.float32, (n,)))
    one = torch.empty(n, dtype=torch.float32, device="cuda")
    sk.score_layers(sL, Q, K, one)
    torch.cuda.synchronize()
    lse.check()
    out.check()
    w = want.cpu().numpy()
    got = out.as_(torch.float32, (n,)).cpu().numpy()
    assert np.array_equal(got.view(np.uint32), w.view(np.uint32)), "two-call all-layer score"
    assert np.array_equal(one.cpu().numpy().view(np.uint32), w.view(np.uint32)), "sk_score_layers"
    g64 = got.astype(np.float64)
    assert np.all(g64 > 0) and np.all(np.isfinite(g64))
    assert abs(g64.sum() - L * Hq * n) <= 1e-4 * L * Hq * n, "row-stochastic invariant"
    del Q, K
    torch.cuda.empty_cache()
