"""The importance score (SpectrumKV paper §4.3 "Importance scores",
Algorithm 1 "score tokens") at the largest sizes its calls accept.

* The token limit, 65535 * 64 = 4,194,240 tokens: the row pass's grid then
  has its full 65535 blocks of 64 queries (4 query heads per KV head, so one
  workgroup holds four heads of one query block).  Checked against the fp64
  oracle on sampled rows of the base-2 lse, on the last 24 columns (cheap:
  they need only the last 24 rows), and by the row-stochastic invariant
  sum_j A_j = H_q * n over all columns.
* The layer limit of the all-layer calls, 65535 layers in one launch per
  pass (the layer is the grid's third dimension): bit for bit what one call
  per layer gives, its lse rows those of the per-layer row pass, and the sum
  over layers against the oracle.

Inputs are seeded fp16 bit patterns: a random sign and mantissa, and an
exponent that puts |x| in [1/8, 2), drawn as raw bytes because normal
variates for a billion elements take half a minute on the host."""

import numpy as np
import pytest
import torch

from oracle import score as OS
import serving_sk_score_amd as sk
from tests.gpu_helpers import Guarded, say, to_dev

pytestmark = pytest.mark.gpu

RTOL = 2e-3
LOG2E = 1.0 / np.log(2.0)   # the row pass reports the log-sum-exp in base 2
MAX_TOKENS = 65535 * 64
MAX_LAYERS = 65535


def _fp16(rng, shape):
    """Seeded fp16 values with |x| in [1/8, 2) and a random sign."""
    bits = np.frombuffer(rng.bytes(2 * int(np.prod(shape))), dtype=np.uint16)
    return ((bits & np.uint16(0x8FFF)) | np.uint16(0x3000)).view(np.float16).reshape(shape)


def _close(got, want, tag):
    rel = np.abs(got - want) / np.abs(want)
    worst = int(np.argmax(rel))
    say(f"{tag}: max rel err {rel.max():.3g}")
    assert rel.max() <= RTOL, f"{tag}: max rel err {rel.max():.3g} at {worst} ({got[worst]} vs {want[worst]})"


def test_score_at_token_limit():
    n, Hq, Hkv, d = MAX_TOKENS, 4, 1, 64
    say("score at the token limit", dict(n=n, Hq=Hq, Hkv=Hkv, d=d))
    rng = np.random.default_rng(2024)
    q = _fp16(rng, (n, Hq, d))
    k = _fp16(rng, (n, Hkv, d))
    shape = sk.Shape(1, Hq, Hkv, d)
    qd, kd = to_dev(q), to_dev(k)
    lse = Guarded(4 * Hq * n)
    sk.score_rowlse(shape, qd, kd, lse.as_(torch.float32, (Hq, n)))
    out = Guarded(4 * n)
    sk.score(shape, qd, kd, out.as_(torch.float32, (n,)), False)
    torch.cuda.synchronize()
    lse.check()
    out.check()
    del qd, kd
    got = out.as_(torch.float32, (n,)).cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(got)) and np.all(got > 0)
    assert abs(got.sum() - Hq * n) <= 1e-4 * Hq * n, "row-stochastic invariant"

    # rows at both ends of the first and last query blocks and in the middle
    rows = np.array([0, 1, 63, 64, n // 2 + 17, n - 65, n - 64, n - 1])
    lse_h = lse.as_(torch.float32, (Hq, n)).cpu().numpy().astype(np.float64)
    for h in (0, Hq - 1):
        say(f"oracle lse, head {h}, rows {rows.tolist()}")
        want = OS.head_row_lse(q[:, h, :], k[:, 0, :], rows) * LOG2E
        err = np.abs(lse_h[h, rows] - want)
        assert err.max() < 1e-3, f"lse head {h}: {err.max():.3g} at row {rows[int(np.argmax(err))]}"

    cols = np.arange(n - 24, n)
    say("oracle last columns", len(cols))
    _close(got[cols], OS.layer_column_sample(q, k, cols), "last columns")


def test_all_layer_launch_at_layer_limit():
    L, n, Hq, Hkv, d = MAX_LAYERS, 3, 4, 1, 64
    say("all-layer score at the layer limit", dict(L=L, n=n, Hq=Hq, Hkv=Hkv, d=d))
    rng = np.random.default_rng(65535)
    qs = _fp16(rng, (L, n, Hq, d))
    ks = _fp16(rng, (L, n, Hkv, d))
    Q, Kt = to_dev(qs), to_dev(ks)
    sL = sk.Shape(L, Hq, Hkv, d)
    got = Guarded(4 * n)
    out = got.as_(torch.float32, (n,))
    sk.score_layers(sL, Q, Kt, out, accumulate=False)
    lse = Guarded(4 * L * Hq * n)
    lseL = lse.as_(torch.float32, (L, Hq, n))
    sk.score_rowlse_layers(sL, Q, Kt, lseL)
    torch.cuda.synchronize()
    got.check()
    lse.check()

    say("one call per layer ...")
    s1 = sk.Shape(1, Hq, Hkv, d)
    want = torch.empty(n, dtype=torch.float32, device="cuda")
    ws = torch.empty(sk.score_workspace_bytes(s1, n), dtype=torch.uint8, device="cuda")
    for layer in range(L):
        sk.score(s1, Q[layer], Kt[layer], want, accumulate=layer > 0, ws=ws)
    probe = [0, 1, L // 2, L - 2, L - 1]
    lse1 = torch.empty((len(probe), Hq, n), dtype=torch.float32, device="cuda")
    for t, layer in enumerate(probe):
        sk.score_rowlse(s1, Q[layer], Kt[layer], lse1[t])
    torch.cuda.synchronize()
    g = out.cpu().numpy()
    assert np.array_equal(g.view(np.uint32), want.cpu().numpy().view(np.uint32)), \
        "all-layer launch differs from one call per layer"
    assert np.array_equal(lseL[probe].cpu().numpy().view(np.uint32),
                          lse1.cpu().numpy().view(np.uint32))

    say("oracle over all layers (fp64) ...")
    _close(g.astype(np.float64), OS.score(qs, ks), "sum over 65535 layers")
