"""Shared helpers of the GPU parity tests (device buffers with canaries,
seeded edge-case rows, progress printing)."""

import sys

import numpy as np
import torch

import serving_sk_score_amd as sk

GUARD = 4096
FILL = 0xA5


def say(*a):
    print("[gpu-test]", *a, flush=True)
    sys.stdout.flush()


def dev():
    return torch.device("cuda", 0)


def to_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev())


class Guarded:
    """A device buffer with 4 KiB canary regions on both sides."""

    def __init__(self, nbytes, fill=FILL):
        self.nbytes = int(nbytes)
        self.fill = fill
        self.raw = torch.full((self.nbytes + 2 * GUARD,), fill, dtype=torch.uint8, device=dev())
        self.bytes = self.raw[GUARD:GUARD + self.nbytes]

    def as_(self, dtype, shape):
        return self.bytes.view(dtype).view(shape)

    def check(self):
        head = self.raw[:GUARD]
        tail = self.raw[GUARD + self.nbytes:]
        assert bool((head == self.fill).all()) and bool((tail == self.fill).all()), "canary overwritten"


def u32(t):
    """int32 torch tensor holding u32 bit patterns -> numpy uint32."""
    return t.cpu().numpy().view(np.uint32)


def edge_rows(rng, rows, d, qmax):
    """fp16 rows with the quantizer's edge cases mixed in: zeros, underflow,
    fp16 extremes, subnormal scales and exact half-step ties."""
    x = (rng.standard_normal((rows, d)) * np.exp(rng.uniform(-6, 3, (rows, 1)))).astype(np.float32)
    kinds = rng.integers(0, 8, size=rows)
    for r in range(rows):
        k = kinds[r]
        if k == 0:
            x[r] = 0.0
        elif k == 1:                                      # underflowing scale
            x[r] = 0.0
            x[r, rng.integers(0, d)] = 2.0 ** -24
        elif k == 2:                                      # largest fp16
            x[r, rng.integers(0, d)] = 65504.0 * rng.choice([-1, 1])
        elif k == 3:                                      # subnormal scale
            x[r] = rng.integers(-qmax * 8, qmax * 8, size=d) * 2.0 ** -24
        elif k == 4:                                      # exact .5 ties: s = 2^e
            e = int(rng.integers(-12, 4))
            m = rng.integers(-qmax, qmax, size=d) + 0.5
            x[r] = m * 2.0 ** e
            x[r, rng.integers(0, d)] = qmax * 2.0 ** e
    return x.astype(np.float16)


def make_kv(seed, L, n, H, d):
    rng = np.random.default_rng(seed)
    K = np.empty((L, n, H, d), dtype=np.float16)
    V = np.empty((L, n, H, d), dtype=np.float16)
    for layer in range(L):
        K[layer] = edge_rows(rng, n * H, d, 127).reshape(n, H, d)
        V[layer] = edge_rows(rng, n * H, d, 7).reshape(n, H, d)
    return K, V


def make_kv_deep(seed, L, n, H, d):
    """K, V for requests with very many layers: seeded normal rows in every
    layer (fast), and the quantizer's edge rows in the first and last layers,
    whose payload offsets are the extreme ones."""
    rng = np.random.default_rng(seed)
    K = (rng.standard_normal((L, n, H, d), dtype=np.float32) * 2.0).astype(np.float16)
    V = (rng.standard_normal((L, n, H, d), dtype=np.float32) * 2.0).astype(np.float16)
    for layer in (0, L - 1):
        K[layer] = edge_rows(rng, n * H, d, 127).reshape(n, H, d)
        V[layer] = edge_rows(rng, n * H, d, 7).reshape(n, H, d)
    return K, V


def tied_scores(seed, n):
    rng = np.random.default_rng(seed)
    s = rng.random(n).astype(np.float32) * 100
    if n > 10:
        idx = rng.integers(0, n, size=n // 5)
        s[idx] = s[idx[0]]                                # a block of exact ties
        s[rng.integers(0, n, size=max(1, n // 50))] = 0.0
    return s


def shape_of(L, Hq, H, d):
    return sk.Shape(L, Hq, H, d)


def fill_layers(cfg, fn, dst, keep=(), threads=16):
    """dst[layer] <- fn(cfg, layer) for every layer, generated on a thread
    pool; returns {layer: host array} for the layers in `keep`."""
    from concurrent.futures import ThreadPoolExecutor
    kept = {}
    L = dst.shape[0]
    with ThreadPoolExecutor(threads) as ex:
        futs = [ex.submit(fn, cfg, layer) for layer in range(L)]
        for layer, f in enumerate(futs):
            a = f.result()
            dst[layer].copy_(torch.from_numpy(a))
            if layer in keep:
                kept[layer] = a
            futs[layer] = None
    return kept
