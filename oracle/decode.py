"""Decode attention over a mixed-precision payload (oracle, float64).  Test
infrastructure only: nothing in the product path imports it.

Sources: SpectrumKV paper (arXiv 2606.08635) §4.2 - the decode worker
dequantizes the received KV and runs attention on it; the Minima-KV page
(mixed-format attention: per-format partial attention states merged by one
globally normalised softmax, no dense shadow) is prior art for computing it
straight from the compressed formats.

Definition, for one layer l and query head h with KV head g = h // (H_q/H_kv):

    o_h   = sum_j softmax_j(q_h . k_hat_j / sqrt(d)) v_hat_j
    lse_h = ln sum_j exp(q_h . k_hat_j / sqrt(d))

over the tokens j that were sent (tiers fp16 / int8 / int4; dropped tokens
take no part), where k_hat, v_hat are the decode-side fp16 rows of the
unpack (the pack oracle's dequantization).  Readings:

1. The attention is over the transferred prefix only; the decode step's own
   new token is the caller's to add, which the returned lse makes possible
   (merge two partial results by their log-sum-exps).
2. No causal mask applies: a decode query follows every prefix token.
3. With no token sent, o = 0 and lse = -inf.
"""

import math

import numpy as np

from . import quant as Q
from .plan import INT4


def layer_attention(payload, amap, plan, layer, H, d, q):
    """q: fp16 [H_q][d] of one layer -> (o float64 [H_q][d], lse float64 [H_q])."""
    k, v = Q.unpack_layer(payload, layer, amap, plan, H, d)
    sent = (np.asarray(amap, dtype=np.uint32) >> 30) <= INT4
    k = k[sent].astype(np.float64)                  # [m][H][d]
    v = v[sent].astype(np.float64)
    q = np.asarray(q, dtype=np.float64)
    Hq = q.shape[0]
    o = np.zeros((Hq, d), dtype=np.float64)
    lse = np.full(Hq, -np.inf, dtype=np.float64)
    if k.shape[0] == 0:
        return o, lse
    for h in range(Hq):
        g = h // (Hq // H)
        s = (k[:, g, :] @ q[h]) / math.sqrt(d)
        m = s.max()
        w = np.exp(s - m)
        o[h] = (w @ v[:, g, :]) / w.sum()
        lse[h] = m + math.log(w.sum())
    return o, lse


def attention(payload, amap, plan, layers, H, d, q):
    """q: fp16 [len(layers)][H_q][d] -> (o [len][H_q][d], lse [len][H_q])."""
    outs, lses = [], []
    for i, layer in enumerate(layers):
        o, lse = layer_attention(payload, amap, plan, layer, H, d, q[i])
        outs.append(o)
        lses.append(lse)
    return np.stack(outs), np.stack(lses)


def merge(o1, lse1, o2, lse2):
    """The attention over the union of two disjoint token sets from the two
    partial results (the log-sum-exp merge)."""
    m = np.maximum(lse1, lse2)
    w1 = np.where(np.isneginf(lse1), 0.0, np.exp(lse1 - m))
    w2 = np.where(np.isneginf(lse2), 0.0, np.exp(lse2 - m))
    tot = w1 + w2
    o = (w1[..., None] * o1 + w2[..., None] * o2) / tot[..., None]
    return o, m + np.log(tot)
