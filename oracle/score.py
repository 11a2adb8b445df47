"""Token importance score (oracle, float64).

Definition (SpectrumKV paper, §4.3 "Importance scores" with lambda = 0, and
Algorithm 1 "score tokens"; the Korean SpectrumKV summary, section on the
importance score, states that the score is the attention a token receives,
aggregated over all heads and layers at prefill):

    score_j = sum_l sum_h sum_{i >= j} softmax_i(q_i . k_j / sqrt(d))_j

where softmax_i runs over the causal keys 0..i of query i, q_i is query head h
and k_j is the key of KV head g = h // (H_q / H_kv) (contiguous GQA groups).

Readings:

* lambda = 0, so I_j = A_j: the recency factor exp(-lambda Delta_j) of §4.3 is
  printed without definitions of Delta_j or lambda.  The lambda > 0 variant
  and the KV-norm fallback of Algorithm 1 are the two functions at the end
  of this module, each with its own reading.
* A sum over heads and layers, not a mean (a positive factor does not change
  the ranking).
* The diagonal i = j is included (a causal softmax includes the token itself).
* Inputs are the post-RoPE fp16 Q and K; no soft-capping, no sliding window.

Arithmetic: fp16 inputs are widened exactly to float64; logits, softmax and
sums are float64.  Rows are processed in blocks of queries only to bound
memory; each row's softmax is computed whole, as the definition states.
"""

import math

import numpy as np

_BLOCK = 512


def _logits(qh, kg, i0, i1, d):
    """s_ij = q_i . k_j / sqrt(d) for queries i0..i1-1 and keys 0..i1-1, with
    the non-causal entries (j > i) set to -inf."""
    s = (qh[i0:i1] @ kg[:i1].T) / math.sqrt(d)
    rows = np.arange(i0, i1)[:, None]
    cols = np.arange(i1)[None, :]
    s[cols > rows] = -np.inf
    return s


def _softmax_rows(s):
    m = s.max(axis=1, keepdims=True)
    p = np.exp(s - m)
    return p / p.sum(axis=1, keepdims=True)


def head_column_sums(qh, kg):
    """A_j for one (query head, key head) pair: sum over i >= j of p_ij.

    qh, kg: [n][d] arrays (any float dtype; widened to float64)."""
    qh = np.asarray(qh, dtype=np.float64)
    kg = np.asarray(kg, dtype=np.float64)
    n, d = qh.shape
    a = np.zeros(n, dtype=np.float64)
    for i0 in range(0, n, _BLOCK):
        i1 = min(n, i0 + _BLOCK)
        p = _softmax_rows(_logits(qh, kg, i0, i1, d))
        a[:i1] += p.sum(axis=0)
    return a


def head_row_lse(qh, kg, rows=None):
    """lse_i = log sum_{j <= i} exp(q_i . k_j / sqrt(d)) for the given rows
    (all rows by default), float64."""
    qh = np.asarray(qh, dtype=np.float64)
    kg = np.asarray(kg, dtype=np.float64)
    n, d = qh.shape
    rows = np.arange(n) if rows is None else np.asarray(rows, dtype=np.int64)
    out = np.empty(len(rows), dtype=np.float64)
    for t, i in enumerate(rows):
        s = (kg[:i + 1] @ qh[i]) / math.sqrt(d)
        m = s.max()
        out[t] = m + math.log(np.exp(s - m).sum())
    return out


def group_of(h, H_q, H_kv):
    """Contiguous GQA grouping: query head h reads KV head h // (H_q / H_kv)."""
    return h // (H_q // H_kv)


def layer_score(q, k, heads=None):
    """Score contribution of one layer, summed over the given query heads
    (all by default).  q: [n][H_q][d], k: [n][H_kv][d]."""
    n, H_q, d = q.shape
    H_kv = k.shape[1]
    heads = range(H_q) if heads is None else heads
    a = np.zeros(n, dtype=np.float64)
    for h in heads:
        a += head_column_sums(q[:, h, :], k[:, group_of(h, H_q, H_kv), :])
    return a


def score(qs, ks):
    """Full score over layers.  qs: [L][n][H_q][d], ks: [L][n][H_kv][d]."""
    total = None
    for q, k in zip(qs, ks):
        a = layer_score(q, k)
        total = a if total is None else total + a
    return total


def layer_column_sample(q, k, cols, heads=None):
    """score contributions of one layer for the listed key positions only.

    Exact same definition as :func:`layer_score`, restricted to columns
    ``cols``; it needs the full rows i >= min(cols), so it is cheap for keys
    near the end of a long sequence."""
    n, H_q, d = q.shape
    H_kv = k.shape[1]
    cols = np.asarray(cols, dtype=np.int64)
    heads = range(H_q) if heads is None else heads
    j0 = int(cols.min())
    out = np.zeros(len(cols), dtype=np.float64)
    for h in heads:
        qh = np.asarray(q[:, h, :], dtype=np.float64)
        kg = np.asarray(k[:, group_of(h, H_q, H_kv), :], dtype=np.float64)
        for i0 in range(j0, n, _BLOCK):
            i1 = min(n, i0 + _BLOCK)
            p = _softmax_rows(_logits(qh, kg, i0, i1, d))
            live = cols < i1                    # p_ij = 0 for j > i
            out[live] += p[:, cols[live]].sum(axis=0)
    return out


def to_fp32(score64):
    """The score handed to tier assignment: fp64 rounded to nearest fp32."""
    return np.asarray(score64, dtype=np.float64).astype(np.float32)


# ---------------------------------------------------------------------------
# Score variants of Algorithm 1 "score tokens"

def recency_weight(a, lam):
    """I_j = A_j * exp(-lambda * Delta_j)   (SpectrumKV §4.3, the printed
    importance formula).

    Reading: the page does not define Delta_j; it is taken as the distance
    of token j from the last prefill token, Delta_j = n - 1 - j, so that
    lambda > 0 favours recent tokens and lambda = 0 gives I_j = A_j.
    float64 throughout."""
    a = np.asarray(a, dtype=np.float64)
    n = a.shape[0]
    delta = (n - 1) - np.arange(n, dtype=np.float64)
    return a * np.exp(-float(lam) * delta)


def kv_norm_score(ks):
    """KV-norm fallback of Algorithm 1 ("compute I_j ... or a KV-norm
    fallback").

    Reading: the page names the fallback without a formula; it is taken as
    the sum over layers and KV heads of the Euclidean norm of the token's
    key vector, score_j = sum_l sum_g ||k[l][j][g]||_2.
    ks: [L][n][H_kv][d] (fp16 widened exactly to float64)."""
    ks = np.asarray(ks, dtype=np.float64)
    L, n, H, d = ks.shape
    out = np.zeros(n, dtype=np.float64)
    for layer in range(L):
        for g in range(H):
            out += np.sqrt((ks[layer, :, g, :] ** 2).sum(axis=1))
    return out

