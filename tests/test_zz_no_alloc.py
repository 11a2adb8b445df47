"""sk_score_noalloc (the allocation-free variant of sk_score, whose workspace
is the library's static per-device scratch) against sk_score with a caller
workspace: bit-identical results (same kernels, same deterministic order) on
consecutive calls, the first at the largest request the scratch holds, the
next on smaller inputs of other shapes (so stale scratch contents from the
previous call are present), and in accumulate mode."""

import numpy as np
import pytest
import torch

import serving_sk_score_amd as sk
from tests.gpu_helpers import say

pytestmark = pytest.mark.gpu


def _inputs(seed, n, Hq, Hkv, d):
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    q = torch.randn((n, Hq, d), generator=g, device="cuda").half()
    k = torch.randn((n, Hkv, d), generator=g, device="cuda").half()
    return q, k


def test_noalloc_matches_workspace_score():
    # (seed, n, Hq, Hkv, d): 32 heads x 131072 tokens needs exactly the 32 MiB
    # of scratch; then smaller requests of other shapes
    cases = [(0, 131072, 32, 8, 128), (1, 5000, 32, 8, 128), (2, 3001, 16, 8, 256),
             (3, 777, 7, 1, 64)]
    for seed, n, Hq, Hkv, d in cases:
        say("noalloc score", dict(n=n, Hq=Hq, Hkv=Hkv, d=d))
        shape = sk.Shape(1, Hq, Hkv, d)
        assert sk.score_workspace_bytes(shape, n) <= sk.SCORE_SCRATCH_BYTES
        q, k = _inputs(seed, n, Hq, Hkv, d)
        want = torch.empty(n, dtype=torch.float32, device="cuda")
        sk.score(shape, q, k, want, False)
        got = torch.full((n,), float("nan"), dtype=torch.float32, device="cuda")
        sk.score_noalloc(shape, q, k, got, False)
        torch.cuda.synchronize()
        w, g = want.cpu().numpy(), got.cpu().numpy()
        assert np.all(np.isfinite(w)) and np.all(w > 0)
        assert np.array_equal(w.view(np.uint32), g.view(np.uint32)), (seed, n)
        # accumulate on top of the previous result, both entry points
        q2, k2 = _inputs(seed + 100, n, Hq, Hkv, d)
        sk.score(shape, q2, k2, want, True)
        sk.score_noalloc(shape, q2, k2, got, True)
        torch.cuda.synchronize()
        assert np.array_equal(want.cpu().numpy().view(np.uint32),
                              got.cpu().numpy().view(np.uint32)), (seed, n, "accumulate")
        del q, k, q2, k2


def test_noalloc_rejects_beyond_scratch():
    shape = sk.Shape(1, 32, 8, 128)
    n = 131073                       # one token past what the scratch holds
    q = torch.zeros((n, 32, 128), dtype=torch.float16, device="cuda")
    k = torch.zeros((n, 8, 128), dtype=torch.float16, device="cuda")
    out = torch.zeros(n, dtype=torch.float32, device="cuda")
    with pytest.raises(sk.SkError) as e:
        sk.score_noalloc(shape, q, k, out)
    assert e.value.status == sk.SK_E_WORKSPACE
    torch.cuda.synchronize()
    assert float(out.abs().max()) == 0.0          # nothing was enqueued
