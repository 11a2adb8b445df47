// Quantize + compaction pack and dequantizing unpack (dense and paged).
//
// SpectrumKV paper, Algorithm 1 "transfer": K and V of every token are
// quantized independently per its precision tier and sent as one payload;
// §4.2: the decode worker only dequantizes.  Quantizer: symmetric absmax with
// one fp16 scale per (layer, token, K|V, KV head) row of d elements.
//
// Mapping to CDNA4: one wavefront owns one (layer, token) and walks its 2*H
// rows (K heads then V heads).  A row of d fp16 values is spread over d/8
// lanes, each holding 8 consecutive elements (one 16-byte load), so a wave
// covers 64/(d/8) rows per step and every global access is a contiguous
// 16/8/4-byte vector per lane.  The absmax is a butterfly max over the lanes
// of a row.  The tier is uniform across the wave, so there is no divergence
// between the fp16 copy and the int8/int4 paths.
//
// Exact arithmetic without a divider: the scale needs fl32(a / qmax) and
// r = fl32(1 / s) per row (see quant8), and each element then uses
//   q0 = x*r,  e = fma(-q0, s, x),  q1 = fma(e, r, q0)
// which equals the correctly rounded quotient fl32(x/s) for every pair of
// fp16 x and fp16 s with |x/s| <= 300 (Markstein's correction step; checked
// exhaustively over all such pairs), so rint(q1) is bit-identical to
// rint(fl32(x/s)) without a per-element division.
#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>

#include "sk_kernels.h"

namespace sk {
namespace {

constexpr int kWaves = 4;  // wavefronts (tokens) per workgroup

struct Segs {
    int64_t cnt[3];
    int64_t oc[3];
    int64_t os[3];
};

Segs make_segs(const TierSeg seg[3]) {
    Segs s;
    for (int t = 0; t < 3; ++t) {
        s.cnt[t] = seg[t].count;
        s.oc[t] = seg[t].off_code;
        s.os[t] = seg[t].off_scale;
    }
    return s;
}

__device__ __forceinline__ float h2f(uint32_t bits16) {
    return __half2float(__ushort_as_half((unsigned short)(bits16 & 0xFFFFu)));
}

template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
    return __builtin_bit_cast(
        float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}

// The maximum over each aligned group of LPR lanes (8, 16 or 32).  Within a
// row of 16 lanes it takes four DPP moves, each folded into its v_max: lane ^
// 1 and lane ^ 2 within a quad, then lane 7 - i of the 8-lane half row and
// lane 15 - i of the row, so that every lane meets every other lane of its
// group; 32-lane groups add one swizzle (lane ^ 16).  Max is exact in any
// order, so the result is that of any other reduction.
template <int LPR>
__device__ __forceinline__ float group_max(float v) {
    static_assert(LPR == 8 || LPR == 16 || LPR == 32, "groups of 8, 16 or 32 lanes");
    v = fmaxf(v, dpp_mov<0xB1>(v));   // quad_perm [1, 0, 3, 2]
    v = fmaxf(v, dpp_mov<0x4E>(v));   // quad_perm [2, 3, 0, 1]
    v = fmaxf(v, dpp_mov<0x141>(v));  // row_half_mirror
    if constexpr (LPR >= 16) v = fmaxf(v, dpp_mov<0x140>(v));  // row_mirror
    if constexpr (LPR >= 32)  // bitmask swizzle: and 0x1F, xor 0x10
        v = fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(
                                                   __builtin_bit_cast(int, v), 0x401F)));
    return v;
}

// Quantize 8 elements of one row whose absmax over the whole row is `a`.
// The row's scale needs fl32(a / QMAX) and fl32(1 / s); neither uses the
// divider: a / QMAX is a multiply by fl32(1 / QMAX) and one fused correction,
// and 1 / s one Newton step from the hardware reciprocal (within one ulp of
// 1 / s); both equal the correctly rounded quotients for every fp16 a and s
// (checked exhaustively on the CPU).  Each code is clamped to [-QMAX, QMAX]
// and rounded to nearest even by adding 1.5 * 2^23, the float whose unit is
// 1 in [2^23, 2^24): the result's low bits then hold the code in two's
// complement (its low byte is the int8 code, its low nibble the int4 one).
// Clamping before rounding gives the same code as after, the bounds being
// integers.
template <int QMAX>
__device__ __forceinline__ void quant8(const float (&x)[8], float a, uint32_t (&cb)[8],
                                       uint32_t& sbits) {
    constexpr float kRq = 1.0f / (float)QMAX;
    constexpr float kMagic = 12582912.0f;  // 1.5 * 2^23
    const float d0 = a * kRq;
    const float s32 = fmaf(fmaf(-d0, (float)QMAX, a), kRq, d0);
    const __half s16 = __float2half_rn(s32);
    sbits = __half_as_ushort(s16);
    const float s = __half2float(s16);
    if (s == 0.0f) {
#pragma unroll
        for (int e = 0; e < 8; ++e) cb[e] = 0u;
        return;
    }
    const float r0 = __builtin_amdgcn_rcpf(s);
    const float r = fmaf(fmaf(-r0, s, 1.0f), r0, r0);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const float q0 = x[e] * r;
        const float err = fmaf(-q0, s, x[e]);
        const float q1 = fmaf(err, r, q0);
        const float c = __builtin_amdgcn_fmed3f(q1, -(float)QMAX, (float)QMAX);
        cb[e] = __float_as_uint(c + kMagic);
    }
}

// The low bytes of four code words as one dword (element e in byte e).
__device__ __forceinline__ uint32_t bytes4(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3) {
    const uint32_t lo = __builtin_amdgcn_perm(c1, c0, 0x0C0C0400u);   // [c0, c1, 0, 0]
    const uint32_t hi = __builtin_amdgcn_perm(c3, c2, 0x04000C0Cu);   // [0, 0, c2, c3]
    return lo | hi;
}

// Eight int4 codes (low nibbles of the code words) as one dword, element 2m
// in bits 0-3 and element 2m+1 in bits 4-7 of byte m.
__device__ __forceinline__ uint32_t nibbles8(const uint32_t (&cb)[8]) {
    uint32_t b0 = bytes4(cb[0], cb[1], cb[2], cb[3]) & 0x0F0F0F0Fu;
    uint32_t b1 = bytes4(cb[4], cb[5], cb[6], cb[7]) & 0x0F0F0F0Fu;
    b0 |= b0 >> 4;  // byte 0: e0 | e1 << 4, byte 2: e2 | e3 << 4
    b1 |= b1 >> 4;
    return __builtin_amdgcn_perm(b1, b0, 0x06040200u);
}

// One lane's 8 elements of a row (a 16-byte piece of fp16) quantized against
// the absmax of the whole row, taken over the row's LPR lanes.
template <int QMAX, int LPR>
__device__ __forceinline__ void quant_piece(const uint4 raw, uint32_t (&q)[8], uint32_t& sbits) {
    float x[8];
    x[0] = h2f(raw.x);
    x[1] = h2f(raw.x >> 16);
    x[2] = h2f(raw.y);
    x[3] = h2f(raw.y >> 16);
    x[4] = h2f(raw.z);
    x[5] = h2f(raw.z >> 16);
    x[6] = h2f(raw.w);
    x[7] = h2f(raw.w >> 16);
    float a = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) a = fmaxf(a, fabsf(x[e]));
    a = group_max<LPR>(a);
    quant8<QMAX>(x, a, q, sbits);
}

// Rows of one (layer, token) handled per wavefront step: a row of D fp16
// values is spread over D/8 lanes (one 16-byte piece each), so a step covers
// 64/(D/8) rows.  A wavefront first issues the loads of NB steps (NB, a power
// of two up to 8, covers all 2H rows of the token when it can), then
// quantizes and stores them, so the loads of a token are in flight together.
// Rows past the token's last one (a partial last batch) re-load that last
// row and are not stored: the loads need no branches.
constexpr int kMaxBatch = 8;

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint4 ld_nt(const uint16_t* p) {
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}
// Payload code loads of 16, 8 and 4 bytes with the non-temporal hint.
__device__ __forceinline__ uint4 ld_nt16(const uint8_t* p) {
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    return make_uint4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ uint2 ld_nt8(const uint8_t* p) {
    const u32x2 v = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
    return make_uint2(v[0], v[1]);
}
__device__ __forceinline__ uint32_t ld_nt4(const uint8_t* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(p));
}
__device__ __forceinline__ void st_nt(uint4 v, void* p) {
    __builtin_nontemporal_store(u32x4{v.x, v.y, v.z, v.w}, reinterpret_cast<u32x4*>(p));
}
__device__ __forceinline__ void st_nt(uint2 v, void* p) {
    __builtin_nontemporal_store(u32x2{v.x, v.y}, reinterpret_cast<u32x2*>(p));
}
__device__ __forceinline__ void st_nt(uint32_t v, void* p) {
    __builtin_nontemporal_store(v, reinterpret_cast<uint32_t*>(p));
}

// Token index of this wavefront, made wave-uniform so that its map entry
// (and block-table entry) are scalar loads.
__device__ __forceinline__ int64_t wave_token() {
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    return (int64_t)blockIdx.x * kWaves + w;
}

template <int D, int NB>
__global__ __launch_bounds__(kWaves * 64) void pack_kernel(
    const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    const uint32_t* __restrict__ map, uint8_t* __restrict__ out, Segs sg, int64_t n,
    int H) {
    constexpr int LPR = D / 8;     // lanes per row
    constexpr int RPP = 64 / LPR;  // rows per step
    const int lane = threadIdx.x & 63;
    const int64_t j = wave_token();
    const int64_t layer = blockIdx.y;
    if (j >= n) return;
    const uint32_t m = map[j];
    const uint32_t t = m >> 30;
    const int64_t slot = m & 0x3FFFFFFFu;
    if (t > 2u || slot >= sg.cnt[t]) return;
    const int part = lane % LPR;
    const int rows = 2 * H;
    const int64_t rowbase = (layer * sg.cnt[t] + slot) * rows;
    const int64_t tokrow = (layer * n + j) * H;

    for (int b0 = 0; b0 < rows; b0 += NB * RPP) {
        uint4 raw[NB];
#pragma unroll
        for (int i = 0; i < NB; ++i) {
            const int r = min(b0 + i * RPP + lane / LPR, rows - 1);
            const uint16_t* src = (r < H ? K : V) + (tokrow + (r < H ? r : r - H)) * D + part * 8;
            raw[i] = ld_nt(src);
        }
        // the tier is uniform across the wavefront
        if (t == 0u) {
#pragma unroll
            for (int i = 0; i < NB; ++i) {
                const int r = b0 + i * RPP + lane / LPR;
                if (r < rows) st_nt(raw[i], out + sg.oc[0] + (rowbase + r) * (2 * D) + part * 16);
            }
        } else if (t == 1u) {
#pragma unroll
            for (int i = 0; i < NB; ++i) {
                const int r = b0 + i * RPP + lane / LPR;
                if (b0 + i * RPP < rows) {  // whole steps: the row group's lanes together
                    uint32_t q[8];
                    uint32_t sbits;
                    quant_piece<127, LPR>(raw[i], q, sbits);
                    uint2 w;
                    w.x = bytes4(q[0], q[1], q[2], q[3]);
                    w.y = bytes4(q[4], q[5], q[6], q[7]);
                    if (r < rows) {
                        const int64_t row = rowbase + r;
                        st_nt(w, out + sg.oc[1] + row * D + part * 8);
                        if (part == 0)
                            *reinterpret_cast<uint16_t*>(out + sg.os[1] + row * 2) =
                                (uint16_t)sbits;
                    }
                }
            }
        } else {
#pragma unroll
            for (int i = 0; i < NB; ++i) {
                const int r = b0 + i * RPP + lane / LPR;
                if (b0 + i * RPP < rows) {
                    uint32_t q[8];
                    uint32_t sbits;
                    quant_piece<7, LPR>(raw[i], q, sbits);
                    const uint32_t w = nibbles8(q);
                    if (r < rows) {
                        const int64_t row = rowbase + r;
                        st_nt(w, out + sg.oc[2] + row * (D / 2) + part * 4);
                        if (part == 0)
                            *reinterpret_cast<uint16_t*>(out + sg.os[2] + row * 2) =
                                (uint16_t)sbits;
                    }
                }
            }
        }
    }
}

// Dequantization to fp16_rne(code * s) with packed fp16 arithmetic: the
// code becomes the exact fp16 integer 1024 + u (u = code + bias, the 0x64
// exponent byte placed above it), the bias is removed exactly, and one
// packed multiply rounds the exact product code * s once (fp16 subnormals
// and overflow to inf as IEEE fp16 multiplication gives them).
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ h2 as_h2(uint32_t u) { return __builtin_bit_cast(h2, u); }
__device__ __forceinline__ uint32_t as_u32(h2 v) { return __builtin_bit_cast(uint32_t, v); }

// Four int8 codes -> two dwords of fp16 pairs (elements 0, 1 and 2, 3).
__device__ __forceinline__ uint2 deq8x4(uint32_t w, h2 s) {
    const uint32_t u = w ^ 0x80808080u;  // code + 128 per byte
    const h2 bias = {(_Float16)-1152.0f, (_Float16)-1152.0f};
    const h2 a = as_h2(__builtin_amdgcn_perm(0x64646464u, u, 0x04010400u)) + bias;
    const h2 b = as_h2(__builtin_amdgcn_perm(0x64646464u, u, 0x04030402u)) + bias;
    return make_uint2(as_u32(a * s), as_u32(b * s));
}

// Eight int4 codes (element 2m in the low nibble of byte m) -> four dwords
// of fp16 pairs in element order: byte m is copied under both exponent
// bytes, the mask keeps its low nibble in the first half (1024 + u) and its
// high nibble in the second (1024 + 16u), and one packed fma with (1, 1/16)
// and (-1032, -72) returns both codes exactly.
__device__ __forceinline__ uint4 deq4x8(uint32_t w, h2 s) {
    const uint32_t u = w ^ 0x88888888u;  // code + 8 per nibble
    const h2 mul = {(_Float16)1.0f, (_Float16)0.0625f};
    const h2 bias = {(_Float16)-1032.0f, (_Float16)-72.0f};
    uint32_t o[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        const uint32_t sel = 0x04000400u | ((uint32_t)m * 0x00010001u);  // [b_m, 0x64, b_m, 0x64]
        const uint32_t t = __builtin_amdgcn_perm(0x64646464u, u, sel) & 0xFFF0FF0Fu;
        o[m] = as_u32(__builtin_elementwise_fma(as_h2(t), mul, bias) * s);
    }
    return make_uint4(o[0], o[1], o[2], o[3]);
}

template <int D, int NB, bool PAGED>
__global__ __launch_bounds__(kWaves * 64) void unpack_kernel(
    const uint8_t* __restrict__ in, const uint32_t* __restrict__ map, Segs sg, int64_t n,
    int H, uint16_t* __restrict__ Ko, uint16_t* __restrict__ Vo,
    const int32_t* __restrict__ block_table, int32_t block_size, int64_t num_blocks) {
    constexpr int LPR = D / 8;
    constexpr int RPP = 64 / LPR;
    const int lane = threadIdx.x & 63;
    const int64_t j = wave_token();
    const int64_t layer = blockIdx.y;
    if (j >= n) return;
    const uint32_t m = map[j];
    const uint32_t t = m >> 30;
    const int64_t slot = m & 0x3FFFFFFFu;
    if (t > 2u || slot >= sg.cnt[t]) return;
    int64_t dstrow;  // row index of head 0 of this token in the output
    if (PAGED) {
        const int64_t blk = block_table[j / block_size];
        if (blk < 0 || blk >= num_blocks) return;
        dstrow = ((layer * num_blocks + blk) * block_size + (j % block_size)) * H;
    } else {
        dstrow = (layer * n + j) * H;
    }
    const int part = lane % LPR;
    const int rows = 2 * H;
    const int64_t rowbase = (layer * sg.cnt[t] + slot) * rows;
    for (int b0 = 0; b0 < rows; b0 += NB * RPP) {
        // codes (and scales) of the whole batch first, then dequantize; the
        // tier is uniform across the wavefront.  Codes are read once
        // (non-temporal loads: 16% faster on a payload cold in HBM than
        // cached ones); the 2-byte scales share lines and stay cached.
        uint4 c[NB];
        uint32_t sc[NB];  // fp16 scale bits
        if (t == 0u) {
#pragma unroll
            for (int i = 0; i < NB; ++i) {
                const int64_t row = rowbase + min(b0 + i * RPP + lane / LPR, rows - 1);
                c[i] = ld_nt16(in + sg.oc[0] + row * (2 * D) + part * 16);
            }
        } else if (t == 1u) {
#pragma unroll
            for (int i = 0; i < NB; ++i) {
                const int64_t row = rowbase + min(b0 + i * RPP + lane / LPR, rows - 1);
                const uint2 w = ld_nt8(in + sg.oc[1] + row * D + part * 8);
                c[i] = make_uint4(w.x, w.y, 0u, 0u);
                sc[i] = *reinterpret_cast<const uint16_t*>(in + sg.os[1] + row * 2);
            }
        } else {
#pragma unroll
            for (int i = 0; i < NB; ++i) {
                const int64_t row = rowbase + min(b0 + i * RPP + lane / LPR, rows - 1);
                c[i] = make_uint4(ld_nt4(in + sg.oc[2] + row * (D / 2) + part * 4), 0u, 0u, 0u);
                sc[i] = *reinterpret_cast<const uint16_t*>(in + sg.os[2] + row * 2);
            }
        }
#pragma unroll
        for (int i = 0; i < NB; ++i) {
            const int r = b0 + i * RPP + lane / LPR;
            uint4 o;
            if (t == 0u) {
                o = c[i];
            } else if (t == 1u) {
                const h2 s = as_h2(sc[i] | (sc[i] << 16));
                const uint2 lo = deq8x4(c[i].x, s);
                const uint2 hi = deq8x4(c[i].y, s);
                o = make_uint4(lo.x, lo.y, hi.x, hi.y);
            } else {
                o = deq4x8(c[i].x, as_h2(sc[i] | (sc[i] << 16)));
            }
            if (r < rows)
                st_nt(o, (r < H ? Ko : Vo) + (dstrow + (r < H ? r : r - H)) * D + part * 8);
        }
    }
}

// Cold-tier upgrade: the fp16 rows of a caller-chosen list of tokens,
// gathered into an upgrade payload (slot i = list entry i, the fp16
// segment's row order) or scattered from it into the dense KV or the paged
// cache.  Same mapping as above: one wavefront per (layer, list entry), its
// 2H rows spread D/8 lanes per row, the loads of NB steps in flight before
// the stores.  A listed token outside [0, n) is skipped.
template <int D, int NB>
__global__ __launch_bounds__(kWaves * 64) void upgrade_pack_kernel(
    const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    const uint32_t* __restrict__ tokens, uint8_t* __restrict__ out, int64_t m, int64_t n,
    int H) {
    constexpr int LPR = D / 8;
    constexpr int RPP = 64 / LPR;
    const int lane = threadIdx.x & 63;
    const int64_t i = wave_token();
    const int64_t layer = blockIdx.y;
    if (i >= m) return;
    const int64_t j = tokens[i];
    if (j >= n) return;
    const int part = lane % LPR;
    const int rows = 2 * H;
    const int64_t rowbase = (layer * m + i) * rows;
    const int64_t tokrow = (layer * n + j) * H;
    for (int b0 = 0; b0 < rows; b0 += NB * RPP) {
        uint4 raw[NB];
#pragma unroll
        for (int s = 0; s < NB; ++s) {
            const int r = min(b0 + s * RPP + lane / LPR, rows - 1);
            raw[s] = ld_nt((r < H ? K : V) + (tokrow + (r < H ? r : r - H)) * D + part * 8);
        }
#pragma unroll
        for (int s = 0; s < NB; ++s) {
            const int r = b0 + s * RPP + lane / LPR;
            if (r < rows) st_nt(raw[s], out + (rowbase + r) * (2 * D) + part * 16);
        }
    }
}

template <int D, int NB, bool PAGED>
__global__ __launch_bounds__(kWaves * 64) void upgrade_unpack_kernel(
    const uint8_t* __restrict__ in, const uint32_t* __restrict__ tokens, int64_t m, int64_t n,
    int H, uint16_t* __restrict__ Ko, uint16_t* __restrict__ Vo,
    const int32_t* __restrict__ block_table, int32_t block_size, int64_t num_blocks) {
    constexpr int LPR = D / 8;
    constexpr int RPP = 64 / LPR;
    const int lane = threadIdx.x & 63;
    const int64_t i = wave_token();
    const int64_t layer = blockIdx.y;
    if (i >= m) return;
    const int64_t j = tokens[i];
    if (j >= n) return;
    int64_t dstrow;
    if (PAGED) {
        const int64_t blk = block_table[j / block_size];
        if (blk < 0 || blk >= num_blocks) return;
        dstrow = ((layer * num_blocks + blk) * block_size + (j % block_size)) * H;
    } else {
        dstrow = (layer * n + j) * H;
    }
    const int part = lane % LPR;
    const int rows = 2 * H;
    const int64_t rowbase = (layer * m + i) * rows;
    for (int b0 = 0; b0 < rows; b0 += NB * RPP) {
        uint4 c[NB];
#pragma unroll
        for (int s = 0; s < NB; ++s) {
            const int64_t row = rowbase + min(b0 + s * RPP + lane / LPR, rows - 1);
            c[s] = *reinterpret_cast<const uint4*>(in + row * (2 * D) + part * 16);
        }
#pragma unroll
        for (int s = 0; s < NB; ++s) {
            const int r = b0 + s * RPP + lane / LPR;
            if (r < rows)
                st_nt(c[s], (r < H ? Ko : Vo) + (dstrow + (r < H ? r : r - H)) * D + part * 8);
        }
    }
}

// Loads batched per wavefront: the power of two (up to kMaxBatch) that
// covers the 2H rows of a token, in steps of 64 / (D/8) rows.
int batch_steps(int d, int H) {
    const int steps = (2 * H + 64 / (d / 8) - 1) / (64 / (d / 8));
    int nb = 1;
    while (nb < steps && nb < kMaxBatch) nb *= 2;
    return nb;
}

template <typename F>
hipError_t dispatch_d(int d, int H, F&& f) {
#define SK_NB_CASES(DV)                                                                   \
    switch (batch_steps(DV, H)) {                                                         \
        case 1: return f(std::integral_constant<int, DV>{}, std::integral_constant<int, 1>{}); \
        case 2: return f(std::integral_constant<int, DV>{}, std::integral_constant<int, 2>{}); \
        case 4: return f(std::integral_constant<int, DV>{}, std::integral_constant<int, 4>{}); \
        default: return f(std::integral_constant<int, DV>{}, std::integral_constant<int, 8>{}); \
    }
    switch (d) {
        case 64: SK_NB_CASES(64)
        case 128: SK_NB_CASES(128)
        case 256: SK_NB_CASES(256)
        default: return hipErrorInvalidValue;
    }
#undef SK_NB_CASES
}

}  // namespace

hipError_t launch_pack(const Dims& s, const TierSeg seg[3], const void* k, const void* v,
                       const uint32_t* map, void* payload, hipStream_t st) {
    const Segs sg = make_segs(seg);
    const dim3 grid((unsigned)((s.n + kWaves - 1) / kWaves), (unsigned)s.L);
    return dispatch_d(s.d, s.Hkv, [&](auto D, auto NB) {
        hipLaunchKernelGGL((pack_kernel<decltype(D)::value, decltype(NB)::value>), grid,
                           dim3(kWaves * 64), 0, st,
                           (const uint16_t*)k, (const uint16_t*)v, map, (uint8_t*)payload, sg,
                           s.n, s.Hkv);
        return hipGetLastError();
    });
}

hipError_t launch_unpack_dense(const Dims& s, const TierSeg seg[3], const void* payload,
                               const uint32_t* map, void* k_out, void* v_out,
                               hipStream_t st) {
    const Segs sg = make_segs(seg);
    const dim3 grid((unsigned)((s.n + kWaves - 1) / kWaves), (unsigned)s.L);
    return dispatch_d(s.d, s.Hkv, [&](auto D, auto NB) {
        hipLaunchKernelGGL((unpack_kernel<decltype(D)::value, decltype(NB)::value, false>), grid,
                           dim3(kWaves * 64), 0, st, (const uint8_t*)payload, map, sg, s.n, s.Hkv,
                           (uint16_t*)k_out, (uint16_t*)v_out, (const int32_t*)nullptr, 1,
                           (int64_t)0);
        return hipGetLastError();
    });
}

hipError_t launch_unpack_paged(const Dims& s, const TierSeg seg[3], const void* payload,
                               const uint32_t* map, void* k_cache, void* v_cache,
                               const int32_t* block_table, int32_t block_size,
                               int64_t num_blocks, hipStream_t st) {
    const Segs sg = make_segs(seg);
    const dim3 grid((unsigned)((s.n + kWaves - 1) / kWaves), (unsigned)s.L);
    return dispatch_d(s.d, s.Hkv, [&](auto D, auto NB) {
        hipLaunchKernelGGL((unpack_kernel<decltype(D)::value, decltype(NB)::value, true>), grid,
                           dim3(kWaves * 64), 0, st, (const uint8_t*)payload, map, sg, s.n, s.Hkv,
                           (uint16_t*)k_cache, (uint16_t*)v_cache, block_table, block_size,
                           num_blocks);
        return hipGetLastError();
    });
}

hipError_t launch_upgrade_pack(const Dims& s, int64_t m, const void* k, const void* v,
                               const uint32_t* tokens, void* payload, hipStream_t st) {
    const dim3 grid((unsigned)((m + kWaves - 1) / kWaves), (unsigned)s.L);
    return dispatch_d(s.d, s.Hkv, [&](auto D, auto NB) {
        hipLaunchKernelGGL((upgrade_pack_kernel<decltype(D)::value, decltype(NB)::value>), grid,
                           dim3(kWaves * 64), 0, st, (const uint16_t*)k, (const uint16_t*)v,
                           tokens, (uint8_t*)payload, m, s.n, s.Hkv);
        return hipGetLastError();
    });
}

hipError_t launch_upgrade_unpack(const Dims& s, int64_t m, const void* payload,
                                 const uint32_t* tokens, void* k_out, void* v_out,
                                 const int32_t* block_table, int32_t block_size,
                                 int64_t num_blocks, hipStream_t st) {
    const dim3 grid((unsigned)((m + kWaves - 1) / kWaves), (unsigned)s.L);
    return dispatch_d(s.d, s.Hkv, [&](auto D, auto NB) {
        if (block_table)
            hipLaunchKernelGGL(
                (upgrade_unpack_kernel<decltype(D)::value, decltype(NB)::value, true>), grid,
                dim3(kWaves * 64), 0, st, (const uint8_t*)payload, tokens, m, s.n, s.Hkv,
                (uint16_t*)k_out, (uint16_t*)v_out, block_table, block_size, num_blocks);
        else
            hipLaunchKernelGGL(
                (upgrade_unpack_kernel<decltype(D)::value, decltype(NB)::value, false>), grid,
                dim3(kWaves * 64), 0, st, (const uint8_t*)payload, tokens, m, s.n, s.Hkv,
                (uint16_t*)k_out, (uint16_t*)v_out, (const int32_t*)nullptr, 1, (int64_t)0);
        return hipGetLastError();
    });
}

}  // namespace sk
