"""Seeded generators for the benchmark's inputs, drawn on the GPU.

Same recipe as :mod:`workloads.gen` (see its docstring), for inputs too large
to draw on the host in reasonable time (the batched mix's queries alone are
73 GB over all layers):

* the bulk N(0, 1) draws come from torch's counter-based Philox generator on
  the device, seeded per (config id, tensor id, layer, request); their values
  therefore differ from the numpy streams of :mod:`workloads.gen`, their
  distribution does not;
* the small per-(layer, KV head) draws - the outlier channels and the sink
  direction - come from exactly the numpy streams :mod:`workloads.gen` uses;
* transforms are applied in float64 and every tensor is rounded once to fp16
  (round to nearest even), as on the host.

Nothing here computes a score, a tier, a quantized code or a payload byte.
"""

import torch

from .configs import Config
from .gen import _TENSOR, rng


def _generator(cfg: Config, tensor: str, layer: int, request: int, device):
    seed = (((cfg.cid * 16 + _TENSOR[tensor]) * 4096 + int(layer)) * 1024 + int(request))
    g = torch.Generator(device=device)
    g.manual_seed(0x5EED0000 + seed)
    return g


def keys(cfg: Config, layer: int, n: int, request: int = 0, device="cuda", out=None):
    """fp16 keys [n][H_kv][d] of one layer, on the device."""
    H, d = cfg.kv_heads, cfg.head_dim
    g = _generator(cfg, "k", layer, request, device)
    if cfg.outliers == 0 and cfg.sink_boost == 1.0:
        k = torch.randn((n, H, d), generator=g, device=device, dtype=torch.float32)
        return _store(k, out)
    k = torch.randn((n, H, d), generator=g, device=device, dtype=torch.float32)
    if cfg.outliers:
        og = rng(cfg, "outlier", layer, request)
        for h in range(H):
            ch = torch.as_tensor(og.choice(d, size=cfg.outliers, replace=False),
                                 device=device)
            k[:, h, ch] = (k[:, h, ch].double() * 10.0).float()
    res = _store(k, out)
    if cfg.sink_boost != 1.0:
        sg = rng(cfg, "sink_dir", layer, request)
        m = min(4, n)
        for h in range(H):
            u = sg.standard_normal(d)
            u /= (u ** 2).sum() ** 0.5
            ut = torch.as_tensor(u, device=device, dtype=torch.float64)
            x = k[:m, h, :].double()
            x = x + (cfg.sink_boost - 1.0) * (x @ ut)[:, None] * ut[None, :]
            res[:m, h, :] = x.half()
    return res


def values(cfg: Config, layer: int, n: int, request: int = 0, device="cuda", out=None):
    """fp16 values [n][H_kv][d] of one layer, on the device."""
    g = _generator(cfg, "v", layer, request, device)
    v = torch.randn((n, cfg.kv_heads, cfg.head_dim), generator=g, device=device,
                    dtype=torch.float32)
    return _store(v, out)


def queries(cfg: Config, layer: int, n: int, request: int = 0, k=None, device="cuda",
            out=None):
    """fp16 queries [n][H_q][d] of one layer, on the device; `k` (this
    layer's fp16 keys) is needed for the recency-biased workloads."""
    Hq, Hkv, d = cfg.q_heads, cfg.kv_heads, cfg.head_dim
    g = _generator(cfg, "q", layer, request, device)
    q = torch.randn((n, Hq, d), generator=g, device=device, dtype=torch.float32)
    if not cfg.recency:
        return _store(q, out)
    if k is None:
        k = keys(cfg, layer, n, request, device)
    w = 64
    csum = torch.zeros((n + 1, Hkv, d), dtype=torch.float64, device=device)
    torch.cumsum(k.double(), dim=0, out=csum[1:])
    idx = torch.arange(n, device=device)
    lo = torch.clamp(idx - (w - 1), min=0)
    hi = torch.clamp(idx + w, max=n)
    window = csum[hi] - csum[lo]                       # [n][Hkv][d]
    del csum
    rep = Hq // Hkv
    res = out if out is not None else torch.empty((n, Hq, d), dtype=torch.float16,
                                                  device=device)
    for h in range(Hq):
        res[:, h, :] = (q[:, h, :].double() + 0.5 * window[:, h // rep, :]).half()
    return res


def _store(x32, out):
    if out is None:
        return x32.half()
    out.copy_(x32)
    return out
