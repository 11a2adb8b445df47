"""Cold-tier upgrade (oracle).  Test infrastructure only: nothing in the
product path imports it.

Source (SpectrumKV paper, arXiv 2606.08635): §4.2 "System architecture in PD
disaggregation" and the cold-tier fetch design paragraph of §8.  A token that
reached the decode worker at int4 or int8 is already there in approximate
form, so a cold-tier fetch only has to raise it to fp16; the approximation
serves attention until the upgrade lands.

Readings where the pages leave a step open:

1. What is sent: the token's fp16 rows.  The pages give the saving as the
   byte difference s16 - s4 but no encoding that realises it, and none of
   fewer than 16 bits per element can restore every fp16 value from its int4
   code: the bucket of code 0, |x| <= s/2, holds thousands of fp16 values.
2. Which tokens: a list chosen by the caller (the pages do not say how the
   decode side picks them).  Repeats are allowed.
3. Upgrade payload layout: the fp16 segment's layout with N = the list length
   and slot = the position in the list: row r = ((l * m + i) * 2 + kv) * H + g,
   2 d bytes each, kv = 0 for K and 1 for V.
4. Decode side: every listed token's rows overwrite that token's rows of the
   dense KV or of the paged cache (the same placement as the unpack).
5. A listed token outside [0, n) is skipped: its payload rows are not
   written and nothing is written for it on the decode side; on the paged
   path, a token whose block id lies outside the pool is skipped as well.
"""

import numpy as np


def upgrade_bytes(L, H, d, m):
    return L * m * 2 * H * 2 * d


def upgrade_pack(K, V, tokens, payload=None):
    """K, V: fp16 [L][n][H][d]; tokens: [m] ints.  Returns the payload
    (uint8 [upgrade_bytes]); rows of skipped tokens keep the bytes of
    ``payload`` (zeros when it is None)."""
    L, n, H, d = K.shape
    tokens = np.asarray(tokens, dtype=np.int64)
    m = tokens.shape[0]
    size = upgrade_bytes(L, H, d, m)
    out = np.zeros(size, dtype=np.uint8) if payload is None else np.array(payload, dtype=np.uint8)
    assert out.size == size
    rows = out.view("<f2").reshape(L, m, 2, H, d)
    for layer in range(L):
        for i, j in enumerate(tokens):
            if 0 <= j < n:
                rows[layer, i, 0] = K[layer, j]
                rows[layer, i, 1] = V[layer, j]
    return out


def _rows(payload, L, H, d, m):
    return np.asarray(payload, dtype=np.uint8).view("<f2").reshape(L, m, 2, H, d)


def upgrade_unpack_dense(payload, tokens, K_out, V_out):
    """Overwrite the listed tokens of K_out, V_out [L][n][H][d] in place."""
    L, n, H, d = K_out.shape
    tokens = np.asarray(tokens, dtype=np.int64)
    rows = _rows(payload, L, H, d, tokens.shape[0])
    for layer in range(L):
        for i, j in enumerate(tokens):
            if 0 <= j < n:
                K_out[layer, j] = rows[layer, i, 0]
                V_out[layer, j] = rows[layer, i, 1]


def upgrade_unpack_paged(payload, tokens, n, block_table, k_cache, v_cache, block_size):
    """Overwrite the listed tokens' rows of k_cache, v_cache
    [L][blocks][block_size][H][d] in place."""
    L, nblocks, _, H, d = k_cache.shape
    tokens = np.asarray(tokens, dtype=np.int64)
    bt = np.asarray(block_table, dtype=np.int64)
    rows = _rows(payload, L, H, d, tokens.shape[0])
    for layer in range(L):
        for i, j in enumerate(tokens):
            if not 0 <= j < n:
                continue
            blk = bt[j // block_size]
            if not 0 <= blk < nblocks:
                continue
            k_cache[layer, blk, j % block_size] = rows[layer, i, 0]
            v_cache[layer, blk, j % block_size] = rows[layer, i, 1]
