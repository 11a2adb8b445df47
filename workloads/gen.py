"""Seeded generators for the synthetic Q/K/V of every workload.

Recipe (stand-in for real-model KV; no dataset or trained weight is used):

* every random stream is ``numpy.random.Generator(PCG64(SeedSequence(0,
  spawn_key=(config id, tensor id, layer, request))))``, so any layer or
  request can be regenerated on its own, on any machine;
* Q, K and V start i.i.d. N(0, 1), drawn in float32, transformed in float64
  where a transform applies, and rounded once to fp16 (round to nearest even);
* ``outliers`` > 0: per (layer, KV head) that many K channels, chosen without
  replacement, are scaled x10 for all tokens (keys are the more
  outlier-sensitive tensor in the SpectrumKV paper's cosine study, Table 8);
* ``sink_boost`` > 1: per (layer, KV head) one random unit direction u; for
  the first four tokens the key component along u is multiplied by the boost
  (k <- k + (boost - 1) (u.k) u);
* ``recency``: query i of head h adds 0.5 x the sum of the keys of its KV head
  at positions j with |i - j| < 64 (a two-sided window, prefix sums in fp64);
* batched mix: request lengths n_r = round(exp(U(ln lo, ln hi))); the paged
  cache's physical blocks are one seeded permutation of all sum_r ceil(n_r/16)
  blocks and request r's block table is the next ceil(n_r/16) entries of it.

Nothing here computes a score, a tier, a quantized code or a payload byte.
"""

import math
from concurrent.futures import ThreadPoolExecutor

import numpy as np

from .configs import Config

_TENSOR = {"q": 0, "k": 1, "v": 2, "sink_dir": 3, "outlier": 4,
           "lengths": 5, "blocks": 6}


def rng(cfg: Config, tensor: str, layer: int = 0, request: int = 0):
    ss = np.random.SeedSequence(0, spawn_key=(cfg.cid, _TENSOR[tensor],
                                              int(layer), int(request)))
    return np.random.Generator(np.random.PCG64(ss))


def _tokens(cfg: Config, n):
    return cfg.tokens if n is None else int(n)


def keys(cfg: Config, layer: int, n=None, request: int = 0) -> np.ndarray:
    """fp16 keys [n][H_kv][d] of one layer."""
    n = _tokens(cfg, n)
    H, d = cfg.kv_heads, cfg.head_dim
    k = rng(cfg, "k", layer, request).standard_normal((n, H, d), dtype=np.float32)
    if cfg.outliers == 0 and cfg.sink_boost == 1.0:
        return k.astype(np.float16)
    k = k.astype(np.float64)
    if cfg.outliers:
        g = rng(cfg, "outlier", layer, request)
        for h in range(H):
            ch = g.choice(d, size=cfg.outliers, replace=False)
            k[:, h, ch] *= 10.0
    if cfg.sink_boost != 1.0:
        g = rng(cfg, "sink_dir", layer, request)
        m = min(4, n)
        for h in range(H):
            u = g.standard_normal(d)
            u /= np.linalg.norm(u)
            c = k[:m, h, :] @ u
            k[:m, h, :] += (cfg.sink_boost - 1.0) * c[:, None] * u[None, :]
    return k.astype(np.float16)


def values(cfg: Config, layer: int, n=None, request: int = 0) -> np.ndarray:
    """fp16 values [n][H_kv][d] of one layer."""
    n = _tokens(cfg, n)
    v = rng(cfg, "v", layer, request).standard_normal(
        (n, cfg.kv_heads, cfg.head_dim), dtype=np.float32)
    return v.astype(np.float16)


def queries(cfg: Config, layer: int, n=None, request: int = 0, k=None) -> np.ndarray:
    """fp16 queries [n][H_q][d] of one layer (post-RoPE stand-ins)."""
    n = _tokens(cfg, n)
    Hq, Hkv, d = cfg.q_heads, cfg.kv_heads, cfg.head_dim
    q = rng(cfg, "q", layer, request).standard_normal((n, Hq, d), dtype=np.float32)
    if not cfg.recency:
        return q.astype(np.float16)
    if k is None:
        k = keys(cfg, layer, n, request)
    q = q.astype(np.float64)
    w = 64
    kk = k.astype(np.float64)
    csum = np.zeros((n + 1, Hkv, d))
    np.cumsum(kk, axis=0, out=csum[1:])
    idx = np.arange(n)
    lo = np.maximum(idx - (w - 1), 0)
    hi = np.minimum(idx + w, n)
    window = csum[hi] - csum[lo]                    # [n][Hkv][d]
    rep = Hq // Hkv
    for h in range(Hq):
        q[:, h, :] += 0.5 * window[:, h // rep, :]
    return q.astype(np.float16)


def request_lengths(cfg: Config):
    """Lengths of the batched mix, log-uniform in [len_lo, len_hi]."""
    g = rng(cfg, "lengths")
    u = g.uniform(math.log(cfg.len_lo), math.log(cfg.len_hi), size=cfg.requests)
    return [int(round(math.exp(x))) for x in u]


def block_tables(cfg: Config, lengths):
    """Per-request int32 block tables over one permuted pool of blocks.

    Returns (tables, num_blocks)."""
    bs = cfg.block_size
    counts = [(n + bs - 1) // bs for n in lengths]
    total = int(sum(counts))
    perm = rng(cfg, "blocks").permutation(total).astype(np.int32)
    tables, off = [], 0
    for c in counts:
        tables.append(perm[off:off + c].copy())
        off += c
    return tables, total


def stacked(cfg: Config, fn, layers=None, n=None, request: int = 0, threads: int = 8):
    """Stack fn(cfg, layer, n, request) over layers -> [L][...] (threaded)."""
    layers = range(cfg.layers) if layers is None else layers
    layers = list(layers)
    first = fn(cfg, layers[0], n, request)
    out = np.empty((len(layers),) + first.shape, dtype=first.dtype)
    out[0] = first

    def one(i):
        out[i] = fn(cfg, layers[i], n, request)

    if len(layers) > 1:
        with ThreadPoolExecutor(max(1, threads)) as ex:
            list(ex.map(one, range(1, len(layers))))
    return out
