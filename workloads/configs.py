"""Workload table.

The shapes follow the evaluated models of the SpectrumKV paper (§5 "Models":
Qwen2.5-7B, Mistral-7B-v0.3, Gemma-2-9B) at long-context lengths, plus a tiny
case that a CPU reference finishes in well under a second and a batched
serving mix that unpacks into a paged cache (PagedAttention-style blocks; the
Minima-KV page describes format-partitioned page tables, here the block size
is 16 tokens).

Fields
------
layers, q_heads, kv_heads, head_dim, tokens : the KV shape (L, H_q, H_kv, d, n).
sinks        : S, the number of leading tokens always kept at fp16.
budget       : b, the normalized transfer budget (fraction of fp16 bytes).
three_tier   : 1 when int4 is allowed (the probe passed), 0 for fp16/int8.
unpack       : "dense" or "paged".
outliers     : number of K channels per (layer, KV head) scaled x10.
sink_boost   : factor applied to the component of keys 0..3 along a random
               unit direction (1 = no boost).
recency      : Gemma-shaped recency bias (queries add 0.5 x the sum of the
               keys within +-63 positions).
requests     : for the batched mix, the number of requests; lengths are drawn
               log-uniformly in [len_lo, len_hi].
budgets      : the budget sweep of the batched mix.
block_size   : tokens per paged-cache block.
"""

from dataclasses import dataclass, field
from typing import Tuple


@dataclass(frozen=True)
class Config:
    name: str
    cid: int
    layers: int
    q_heads: int
    kv_heads: int
    head_dim: int
    tokens: int
    sinks: int
    budget: float
    three_tier: int
    unpack: str = "dense"
    outliers: int = 0
    sink_boost: float = 1.0
    recency: bool = False
    requests: int = 0
    len_lo: int = 0
    len_hi: int = 0
    budgets: Tuple[float, ...] = field(default_factory=tuple)
    block_size: int = 16

    @property
    def shape(self):
        return (self.layers, self.q_heads, self.kv_heads, self.head_dim)


CONFIGS = {
    "tiny": Config(
        name="tiny", cid=0, layers=1, q_heads=4, kv_heads=2, head_dim=64,
        tokens=256, sinks=4, budget=0.5, three_tier=1, unpack="dense",
        sink_boost=8.0),
    "mistral7b": Config(
        name="mistral7b", cid=1, layers=32, q_heads=32, kv_heads=8,
        head_dim=128, tokens=8192, sinks=4, budget=0.5, three_tier=1,
        unpack="dense", outliers=4, sink_boost=8.0),
    "qwen25_7b_2tier": Config(
        name="qwen25_7b_2tier", cid=2, layers=28, q_heads=28, kv_heads=4,
        head_dim=128, tokens=32768, sinks=4, budget=0.6, three_tier=0,
        unpack="dense", outliers=4, sink_boost=8.0),
    "gemma2_9b": Config(
        name="gemma2_9b", cid=3, layers=42, q_heads=16, kv_heads=8,
        head_dim=256, tokens=32768, sinks=4, budget=0.3, three_tier=1,
        unpack="dense", recency=True),
    "batched_mix": Config(
        name="batched_mix", cid=4, layers=32, q_heads=32, kv_heads=8,
        head_dim=128, tokens=0, sinks=4, budget=0.5, three_tier=1,
        unpack="paged", outliers=4, sink_boost=8.0, requests=16,
        len_lo=1024, len_hi=65536, budgets=(0.3, 0.5, 0.7), block_size=16),
}


def get_config(name: str) -> Config:
    try:
        return CONFIGS[name]
    except KeyError:
        raise KeyError(f"unknown workload {name!r}; known: {sorted(CONFIGS)}")
