"""Quantizer, pack and unpack (oracle, IEEE fp32/fp16 arithmetic).

Sources (SpectrumKV paper, arXiv 2606.08635):

* Algorithm 1, "transfer": keys and values are quantized independently
  according to the precision map and sent as one mixed-precision payload.
* §2.1: int4 carries a quarter and int8 half of the fp16 bytes (c(4) = 1/4,
  c(8) = 1/2), so int4 codes are 4 bits and int8 codes 8 bits per element.
* §4.2: the decode worker only dequantizes (a table-lookup-cheap step).

The quantizer itself is the symmetric absmax per-row scheme: one fp16 scale
per (layer, token, K|V, KV head) row of d elements.

Readings:

1. a = max_i |x_i| (exact in fp32); s32 = fl32(a / qmax) with a correctly
   rounded fp32 division (qmax = 127 for int8, 7 for int4); s16 = the fp16
   nearest to s32 (ties to even).  Codes are computed from the stored fp16
   scale so that encoder and decoder agree.
2. q_i = clamp(rint_even(fl32(x_i / s16)), -qmax, qmax); the range is
   symmetric (no -128 / -8 code).
3. a = 0, or s16 rounding to 0 (underflow), gives an all-zero row of codes.
4. int8 codes are two's complement bytes; int4 codes are two's complement
   nibbles, element 2m in bits 0-3 and element 2m+1 in bits 4-7 of byte m.
5. Dequantization: x_hat_i = fp16_rne(fp32(q_i) * fp32(s16)) - the product is
   exact in fp32, so there is exactly one rounding.  fp16 rows are copied.
6. Payload layout: five segments c16 | c8 | c4 | s8 | s4 (offsets from the
   plan), row r = ((l * N_t + slot) * 2 + kv) * H_kv + g within each tier's
   segments, kv = 0 for K and 1 for V; scales are little-endian fp16.
7. Paged output: token j of a request goes to
   cache[l][block_table[j // block_size]][j % block_size][g][:]; cache rows
   that hold no token of the request are left untouched.
"""

import numpy as np

from .plan import FP16, INT8, INT4

QMAX = {INT8: 127, INT4: 7}
_SLOT_MASK = (1 << 30) - 1


def quantize_rows(x, qmax):
    """x: fp16 [..., d] -> (codes int8 [..., d], scale fp16 [...])."""
    x32 = np.asarray(x, dtype=np.float16).astype(np.float32)
    a = np.max(np.abs(x32), axis=-1)
    s32 = a / np.float32(qmax)                      # IEEE fp32 division
    s16 = s32.astype(np.float16)                    # round to nearest even
    sdiv = s16.astype(np.float32)
    live = sdiv != 0
    with np.errstate(divide="ignore", invalid="ignore"):
        t = x32 / np.where(live, sdiv, np.float32(1))[..., None]
    q = np.clip(np.rint(t), -qmax, qmax)
    q = np.where(live[..., None], q, 0)
    return q.astype(np.int8), s16


def dequantize_rows(codes, s16):
    """codes int [..., d], s16 fp16 [...] -> fp16 [..., d] (one rounding)."""
    prod = np.asarray(codes).astype(np.float32) * np.asarray(s16, dtype=np.float16).astype(np.float32)[..., None]
    with np.errstate(over="ignore"):     # |q s| above 65504 rounds to +-inf, as IEEE fp16 does
        return prod.astype(np.float16)


def encode_int4(codes):
    """int8 codes in [-7, 7], [..., d] -> packed bytes [..., d/2]."""
    nib = (np.asarray(codes).astype(np.int16) & 0xF).astype(np.uint8)
    return (nib[..., 0::2] | (nib[..., 1::2] << 4)).astype(np.uint8)


def decode_int4(packed):
    """packed bytes [..., d/2] -> int8 codes [..., d] (sign-extended)."""
    p = np.asarray(packed, dtype=np.uint8)
    lo = (p & 0xF).astype(np.int16)
    hi = (p >> 4).astype(np.int16)
    lo = np.where(lo >= 8, lo - 16, lo)
    hi = np.where(hi >= 8, hi - 16, hi)
    out = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), dtype=np.int8)
    out[..., 0::2] = lo
    out[..., 1::2] = hi
    return out


def _tiers(amap):
    amap = np.asarray(amap, dtype=np.uint32)
    return (amap >> 30).astype(np.int64), (amap & _SLOT_MASK).astype(np.int64)


def _counts(plan):
    return {FP16: plan.n16, INT8: plan.n8, INT4: plan.n4}


def _segments(plan):
    return {FP16: (plan.off_c16, None), INT8: (plan.off_c8, plan.off_s8),
            INT4: (plan.off_c4, plan.off_s4)}


def _row_bytes(t, d):
    return {FP16: 2 * d, INT8: d, INT4: d // 2}[t]


def pack_layer(k, v, layer, amap, plan):
    """Bytes of one layer.  k, v: fp16 [n][H][d].

    Returns a list of (payload offset, uint8 array) pieces."""
    n, H, d = k.shape
    tier, slot = _tiers(amap)
    cnt = _counts(plan)
    seg = _segments(plan)
    pieces = []
    for t in (FP16, INT8, INT4):
        toks = np.nonzero(tier == t)[0]
        N = cnt[t]
        assert len(toks) == N
        rows = np.empty((N, 2, H, d), dtype=np.float16)
        rows[slot[toks], 0] = k[toks]
        rows[slot[toks], 1] = v[toks]
        rb = _row_bytes(t, d)
        code_off = seg[t][0] + layer * N * 2 * H * rb
        if t == FP16:
            pieces.append((code_off, rows.astype("<f2").view(np.uint8).reshape(-1)))
            continue
        codes, s16 = quantize_rows(rows, QMAX[t])
        data = codes.view(np.uint8) if t == INT8 else encode_int4(codes)
        pieces.append((code_off, np.ascontiguousarray(data).reshape(-1)))
        sc_off = seg[t][1] + layer * N * 2 * H * 2
        pieces.append((sc_off, s16.astype("<f2").view(np.uint8).reshape(-1)))
    return pieces


def pack(K, V, amap, plan):
    """K, V: fp16 [L][n][H][d] -> payload uint8 [plan.payload_bytes]."""
    out = np.zeros(plan.payload_bytes, dtype=np.uint8)
    written = np.zeros(plan.payload_bytes, dtype=bool)
    for layer in range(K.shape[0]):
        for off, data in pack_layer(K[layer], V[layer], layer, amap, plan):
            out[off:off + data.size] = data
            written[off:off + data.size] = True
    assert written.all(), "layout leaves a byte unwritten"
    return out


def unpack_layer(payload, layer, amap, plan, H, d):
    """Dequantized fp16 K, V [n][H][d] of one layer."""
    payload = np.asarray(payload, dtype=np.uint8)
    tier, slot = _tiers(amap)
    n = tier.shape[0]
    cnt = _counts(plan)
    seg = _segments(plan)
    k = np.empty((n, H, d), dtype=np.float16)
    v = np.empty((n, H, d), dtype=np.float16)
    for t in (FP16, INT8, INT4):
        N = cnt[t]
        toks = np.nonzero(tier == t)[0]
        rb = _row_bytes(t, d)
        code_off = seg[t][0] + layer * N * 2 * H * rb
        raw = payload[code_off:code_off + N * 2 * H * rb].reshape(N, 2, H, rb)
        if t == FP16:
            rows = raw.copy().view("<f2").astype(np.float16)
        else:
            sc_off = seg[t][1] + layer * N * 2 * H * 2
            s16 = payload[sc_off:sc_off + N * 2 * H * 2].copy().view("<f2").reshape(N, 2, H)
            codes = raw.view(np.int8) if t == INT8 else decode_int4(raw)
            rows = dequantize_rows(codes, s16)
        k[toks] = rows[slot[toks], 0]
        v[toks] = rows[slot[toks], 1]
    return k, v


def unpack_dense(payload, amap, plan, L, H, d, K=None, V=None):
    """Dequantized K, V [L][n][H][d].  Rows of dropped tokens (tier 3) are
    not written: they keep the contents of K, V when given."""
    n = len(amap)
    K = np.empty((L, n, H, d), dtype=np.float16) if K is None else K
    V = np.empty((L, n, H, d), dtype=np.float16) if V is None else V
    sent = _tiers(amap)[0] <= INT4
    for layer in range(L):
        k, v = unpack_layer(payload, layer, amap, plan, H, d)
        K[layer, sent] = k[sent]
        V[layer, sent] = v[sent]
    return K, V


def unpack_paged(payload, amap, plan, L, H, d, block_table, k_cache, v_cache,
                 block_size=16):
    """Write the request's rows into k_cache / v_cache [L][blocks][bs][H][d]
    in place (reading 7)."""
    n = len(amap)
    bt = np.asarray(block_table, dtype=np.int64)
    j = np.nonzero(_tiers(amap)[0] <= INT4)[0]          # dropped tokens: untouched
    blk = bt[j // block_size]
    pos = j % block_size
    for layer in range(L):
        k, v = unpack_layer(payload, layer, amap, plan, H, d)
        k_cache[layer, blk, pos] = k[j]
        v_cache[layer, blk, pos] = v[j]
