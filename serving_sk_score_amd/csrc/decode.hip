// Decode attention straight from the mixed-precision payload: the decode
// worker's attention over the transferred prefix (SpectrumKV paper, §4.2)
// without the dense unpack.  Every K/V element is dequantized while it is
// loaded, to exactly the fp16 value the unpack would write
// (fp16_rne(code * scale)), and the per-tier partial results are merged by
// their log-sum-exps (the Minima-KV page's per-format partial states are the
// prior art for that merge).
//
// The work is bound by reading the payload (about half the fp16 bytes at
// b = 0.5).  Per element the vector ALUs only dequantize: fp16 bit patterns
// 1024 + u (u = code + 128 for int8, code + 8 for int4) are built with
// v_perm_b32 (int8) or v_and_or_b32 (int4, two channels i and i + 4 at a
// time), the bias is removed with one packed fp16 add (or fma) and the
// scale applied with one packed fp16 multiply (exact integers, one
// correctly rounded product).  The contractions go to the matrix cores.
// Two bodies compute the same values:
//   - partial_mfma (d = 128, and d = 256 except fp16 rows): both q.k and
//     p.V on v_mfma_f32_16x16x32_f16, the probabilities kept in the lanes
//     that computed them, V read back from LDS with the transposing read
//     (described at that function);
//   - partial_body (d = 64, and fp16 rows at d = 256): q.k as S^T = K Q^T on
//     v_mfma_f32_32x32x16_f16, 32 tokens per row block and the query
//     group's G = H_q/H_kv heads as columns (held in VGPRs; the other
//     32 - G columns are zero), lane l loading token l%32 and half l/32 of
//     the head dimension (the A operand layout when the contraction runs
//     over the dims of each half in turn); p.V on the vector ALUs with
//     v_dot2_f32_f16 over token pairs, the dequantized V rows staged in LDS
//     so that lanes own channel pairs.
// Softmax is online per head across the chunk's 64-token tiles, base 2
// (c2 = log2(e)/sqrt(d)).  One wavefront per (layer, KV head, tier, chunk of
// 64*T slots) writes (m, l, o[d]) per query head; merge_kernel combines the
// chunks of every tier of a (layer, head) in a fixed order.
#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>

#include <math.h>

#include <atomic>
#include <type_traits>

#include "sk_kernels.h"

namespace sk {
namespace {

typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ h2 as_h2(uint32_t u) { return __builtin_bit_cast(h2, u); }
__device__ __forceinline__ uint32_t as_u32(h2 v) { return __builtin_bit_cast(uint32_t, v); }

// Cached 16-byte load: one load instruction reads 32 bytes of each of 32
// rows, so a row's 128-byte line is consumed by consecutive instructions and
// must stay cached between them.
// Buffer resource over `bytes` bytes at `base` for raw loads: the hardware
// range check returns zeros for any load at or past the end.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                             0x00020000);
}

__device__ __forceinline__ u32x4 ld16(const uint8_t* p) {
    return *reinterpret_cast<const u32x4*>(p);
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m, 64));
    return v;
}

// Four int8 codes -> two dwords of fp16 pairs fp16_rne(code * s).
__device__ __forceinline__ void deq8(uint32_t w, h2 s, uint32_t& lo, uint32_t& hi) {
    const uint32_t u = w ^ 0x80808080u;  // code + 128 per byte
    const h2 bias = {(_Float16)-1152.0f, (_Float16)-1152.0f};
    const h2 a = as_h2(__builtin_amdgcn_perm(0x64646464u, u, 0x04010400u)) + bias;
    const h2 b = as_h2(__builtin_amdgcn_perm(0x64646464u, u, 0x04030402u)) + bias;
    lo = as_u32(a * s);
    hi = as_u32(b * s);
}

// (w & m) ^ c in one v_bitop3_b32 (truth table 0x6A: bit (a << 2 | b << 1
// | c) of the table is the result for operand bits a, b, c).
__device__ __forceinline__ uint32_t and_xor(uint32_t w, uint32_t m, uint32_t c) {
    return __builtin_amdgcn_bitop3_b32(w, m, c, 0x6A);
}

// Eight int4 codes (element 2m in the low nibble of byte m) -> four dwords
// of fp16 pairs, in the order (e0, e4), (e1, e5), (e2, e6), (e3, e7): the
// pair of elements i and i + 4 sits at bits 4i and 4i + 16 of the dword, so
// one mask per pair places both nibbles under the 0x64 exponent bytes (bits
// 0-3 for even i after a shift by 8 for i >= 2), and the same instruction
// flips each nibble's top bit, turning the two's complement code into
// u = code + 8: ((w ^ 0x88888888) & m) | 0x64006400 equals
// (w & m) ^ ((0x88888888 & m) | 0x64006400) for every w, since the exponent
// bits lie outside the mask (an xor there sets them as the or does, and
// inside it the and and the xor commute).  The low nibble of a byte
// gives 1024 + u, the high one 1024 + 16u, whose packed fma with 1/16
// (exact) and -72 returns u - 8 in one step.  The caller keeps track of that
// channel order (q for K, the output for V).
__device__ __forceinline__ void deq4(uint32_t w, h2 s, uint32_t (&o)[4]) {
    const uint32_t w2 = w >> 8;
    const h2 lo_bias = {(_Float16)-1032.0f, (_Float16)-1032.0f};
    const h2 hi_mul = {(_Float16)0.0625f, (_Float16)0.0625f};
    const h2 hi_bias = {(_Float16)-72.0f, (_Float16)-72.0f};
    const h2 a0 = as_h2(and_xor(w, 0x000F000Fu, 0x64086408u)) + lo_bias;    // e0, e4
    const h2 a1 = __builtin_elementwise_fma(as_h2(and_xor(w, 0x00F000F0u, 0x64806480u)), hi_mul,
                                            hi_bias);                          // e1, e5
    const h2 a2 = as_h2(and_xor(w2, 0x000F000Fu, 0x64086408u)) + lo_bias;   // e2, e6
    const h2 a3 = __builtin_elementwise_fma(as_h2(and_xor(w2, 0x00F000F0u, 0x64806480u)), hi_mul,
                                            hi_bias);                          // e3, e7
    o[0] = as_u32(a0 * s);
    o[1] = as_u32(a1 * s);
    o[2] = as_u32(a2 * s);
    o[3] = as_u32(a3 * s);
}

// Channel of the first element of fp16 pair w of a dequantized row (the
// second is this + 1, or + 4 for int4, whose pairs come in deq4's order).
template <int TIER>
__device__ __forceinline__ int pair_channel(int w) {
    return TIER == 2 ? 8 * (w >> 2) + (w & 3) : 2 * w;
}
template <int TIER>
constexpr int pair_step() { return TIER == 2 ? 4 : 1; }

// Row bytes per tier and the number of fp16 pairs one 16-byte piece yields.
template <int D, int TIER>
struct Tier {
    static constexpr int RB = TIER == 0 ? 2 * D : (TIER == 1 ? D : D / 2);
    static constexpr int NP = RB / 16;                          // pieces per row
    static constexpr int PPP = TIER == 0 ? 4 : (TIER == 1 ? 8 : 16);  // pairs per piece
};

template <int D, int TIER>
__device__ __forceinline__ void piece_pairs(u32x4 r, h2 s, uint32_t (&pr)[Tier<D, TIER>::PPP]) {
    if constexpr (TIER == 0) {
        pr[0] = r.x;
        pr[1] = r.y;
        pr[2] = r.z;
        pr[3] = r.w;
    } else if constexpr (TIER == 1) {
        deq8(r.x, s, pr[0], pr[1]);
        deq8(r.y, s, pr[2], pr[3]);
        deq8(r.z, s, pr[4], pr[5]);
        deq8(r.w, s, pr[6], pr[7]);
    } else {
        uint32_t t[4];
        deq4(r.x, s, t);
        pr[0] = t[0]; pr[1] = t[1]; pr[2] = t[2]; pr[3] = t[3];
        deq4(r.y, s, t);
        pr[4] = t[0]; pr[5] = t[1]; pr[6] = t[2]; pr[7] = t[3];
        deq4(r.z, s, t);
        pr[8] = t[0]; pr[9] = t[1]; pr[10] = t[2]; pr[11] = t[3];
        deq4(r.w, s, t);
        pr[12] = t[0]; pr[13] = t[1]; pr[14] = t[2]; pr[15] = t[3];
    }
}

struct TierArgs {
    int64_t off_code, off_scale;  // the tier's segments
    int64_t N;                    // tokens in the tier
    int64_t chunk_base;           // first global chunk index of the tier
};

struct PartialArgs {
    const uint8_t* payload;
    TierArgs tier[3];
    int64_t cend[3];              // cumulative chunk counts: tier t owns [cend[t-1], cend[t])
    int H, G, Hq;
    int layer0;
    const uint16_t* q;            // [nl][Hq][D]
    float* part;                  // [nl][Hq][NC][D + 2]
    int64_t NC;                   // chunks over all tiers
    int T;                        // 64-token tiles per chunk
    float c2;                     // log2(e) / sqrt(D)
};

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef float f16v __attribute__((ext_vector_type(16)));

__device__ __forceinline__ h8 pairs_h8(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
    u32x4 v = {a, b, c, d};
    return __builtin_bit_cast(h8, v);
}

// The K and V half rows of one 32-token block as loaded by one lane, with
// their scales.
template <int NPH>
struct BlockRegs {
    u32x4 k[NPH], v[NPH];
    uint16_t sk, sv;  // fp16 scale bits
};

template <int D>
constexpr int lds_pitch() { return D / 2 + 4; }  // V row pitch in dwords

template <int D, int TIER, int GM>
__device__ __forceinline__ void partial_body(const PartialArgs& a, const TierArgs& ta,
                                             int64_t chunk, uint32_t* vt, uint32_t* pp) {
    using TI = Tier<D, TIER>;
    constexpr int CP = D / 2;                     // fp16 pairs per row
    constexpr int HP = CP / 2;                    // pairs per half row
    constexpr int NPH = TI::NP / 2;               // 16-byte pieces per half row
    constexpr int KK = D / 16;                    // MFMAs per 32-token block
    constexpr int LPT = CP < 64 ? CP : 64;        // lanes per token group in p.V
    constexpr int TG = 64 / LPT;                  // token groups (2 for d = 64)
    constexpr int DWL = CP / LPT;                 // pairs owned per lane in p.V
    constexpr int PITCH = lds_pitch<D>();         // vt: [64 tokens (32 at d = 256)][PITCH] dwords
    constexpr bool kSplitV = D == 256;            // V through LDS one block at a time
    static_assert(GM <= 32, "query group wider than the MFMA tile");
    // pp: [32 token pairs][GM heads] fp16 probability pairs

    const int lane = threadIdx.x;
    const int r = lane & 31;   // token within a 32-token block; head column of S^T
    const int hb = lane >> 5;  // half of the head dimension
    const int g = blockIdx.y;
    const int li = blockIdx.z;
    const int64_t layer = a.layer0 + li;
    const int G = a.G;
    const int64_t N = ta.N;

    // Q^T as the B operand: column r = head g*G + r (zero past G), rows = the
    // dims of half hb, 8 per MFMA
    h8 qb[KK];
    {
        const uint32_t* qrow = reinterpret_cast<const uint32_t*>(a.q) +
                               ((int64_t)li * a.Hq + (int64_t)g * G + (r < G ? r : 0)) * CP +
                               hb * HP;
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
            u32x4 v = *reinterpret_cast<const u32x4*>(qrow + 4 * kk);
            if (r >= G) v = u32x4{0u, 0u, 0u, 0u};
            if constexpr (TIER == 2) {
                // dims 0..7 of the group in deq4's order 0, 4, 1, 5, 2, 6, 3, 7
                v = u32x4{__builtin_amdgcn_perm(v.z, v.x, 0x05040100u),
                          __builtin_amdgcn_perm(v.z, v.x, 0x07060302u),
                          __builtin_amdgcn_perm(v.w, v.y, 0x05040100u),
                          __builtin_amdgcn_perm(v.w, v.y, 0x07060302u)};
            }
            qb[kk] = __builtin_bit_cast(h8, v);
        }
    }

    const uint8_t* code = a.payload + ta.off_code + hb * (TI::RB / 2);
    const uint16_t* scale = reinterpret_cast<const uint16_t*>(a.payload + ta.off_scale);
    // issue the loads of the 32-token block starting at slot b0 (slots past
    // the tier's end re-load its last token; they are masked later)
    auto load_block = [&](BlockRegs<NPH>& R, int64_t b0) {
        const int64_t slot = b0 + r < N ? b0 + r : N - 1;
        const int64_t rowK = ((layer * N + slot) * 2) * a.H + g;
        const int64_t rowV = rowK + a.H;
        const uint8_t* kp = code + rowK * TI::RB;
        const uint8_t* vp = code + rowV * TI::RB;
#pragma unroll
        for (int i = 0; i < NPH; ++i) {
            R.k[i] = ld16(kp + i * 16);
            R.v[i] = ld16(vp + i * 16);
        }
        if constexpr (TIER != 0) {
            R.sk = scale[rowK];
            R.sv = scale[rowV];
        }
    };
    // an ordering point: nothing computed from R may move above it, so the
    // loads issued just before it are in flight while R is used
    auto pin = [&](BlockRegs<NPH>& R) {
#pragma unroll
        for (int i = 0; i < NPH; ++i) asm volatile("" : "+v"(R.k[i]), "+v"(R.v[i]));
        if constexpr (TIER != 0) asm volatile("" : "+v"(R.sk), "+v"(R.sv));
    };
    // dequantize a block's K into the S^T MFMAs, one 16-byte piece at a time
    // (each piece's fp16 pairs feed their MFMAs right away, so the whole
    // dequantized half row is never held)
    auto k_block = [&](const BlockRegs<NPH>& R, f16v& c) {
        h2 sk2 = {(_Float16)1.0f, (_Float16)1.0f};
        if constexpr (TIER != 0) {
            // consumed here, not earlier: a wait for a prefetched block's
            // scale would also wait for every load issued before it
            uint32_t ks = R.sk;
            asm volatile("" : "+v"(ks));
            sk2 = as_h2(ks | (ks << 16));
        }
        c = f16v{};
#pragma unroll
        for (int i = 0; i < NPH; ++i) {
            uint32_t pr[TI::PPP];
            piece_pairs<D, TIER>(R.k[i], sk2, pr);
#pragma unroll
            for (int j = 0; j < TI::PPP / 4; ++j)
                c = __builtin_amdgcn_mfma_f32_32x32x16_f16(
                    pairs_h8(pr[4 * j], pr[4 * j + 1], pr[4 * j + 2], pr[4 * j + 3]),
                    qb[i * (TI::PPP / 4) + j], c, 0, 0, 0);
        }
    };
    // dequantize a block's V into the LDS rows (rows of slots past the
    // tier's end hold a copy of its last token; their probabilities are
    // exactly 0)
    auto v_block = [&](const BlockRegs<NPH>& R, int row0) {
        h2 sv2 = {(_Float16)1.0f, (_Float16)1.0f};
        if constexpr (TIER != 0) {
            uint32_t vs = R.sv;
            asm volatile("" : "+v"(vs));
            sv2 = as_h2(vs | (vs << 16));
        }
        uint32_t* vrow = &vt[(row0 + r) * PITCH + hb * HP];
#pragma unroll
        for (int i = 0; i < NPH; ++i) {
            uint32_t pv[TI::PPP];
            piece_pairs<D, TIER>(R.v[i], sv2, pv);
#pragma unroll
            for (int e = 0; e < TI::PPP; e += 4)
                *reinterpret_cast<u32x4*>(vrow + i * TI::PPP + e) =
                    u32x4{pv[e], pv[e + 1], pv[e + 2], pv[e + 3]};
        }
    };

    float m = -INFINITY, lsum = 0.0f;  // of head column r, scaled (base-2) domain
    float o[GM][DWL][2];
#pragma unroll
    for (int h = 0; h < GM; ++h)
#pragma unroll
        for (int k = 0; k < DWL; ++k) o[h][k][0] = o[h][k][1] = 0.0f;

    BlockRegs<NPH> A, B;
    // p.V of token pairs [tp0, tp0 + NTP) of the tile, whose V rows are in
    // LDS from row vr0 on: lanes own channel pairs, tokens two at a time
    auto pv_rows = [&](auto ntp, int tp0, int vr0) {
        constexpr int NTP = decltype(ntp)::value;
        const int tg = TG > 1 ? lane / LPT : 0;
        const int wl = TG > 1 ? lane % LPT : lane;
#pragma unroll
        for (int it = 0; it < NTP / TG; ++it) {
            const int tp = it * TG + tg;          // token pair within the rows
            uint32_t pw[GM];
#pragma unroll
            for (int h = 0; h < GM; ++h) pw[h] = pp[(tp0 + tp) * GM + h];
#pragma unroll
            for (int k = 0; k < DWL; ++k) {
                const int w = wl + k * LPT;
                const uint32_t x = vt[(vr0 + 2 * tp) * PITCH + w];
                const uint32_t y = vt[(vr0 + 2 * tp + 1) * PITCH + w];
                const h2 a0 = as_h2(__builtin_amdgcn_perm(y, x, 0x05040100u));
                const h2 a1 = as_h2(__builtin_amdgcn_perm(y, x, 0x07060302u));
#pragma unroll
                for (int h = 0; h < GM; ++h) {
                    o[h][k][0] = __builtin_amdgcn_fdot2(a0, as_h2(pw[h]), o[h][k][0], false);
                    o[h][k][1] = __builtin_amdgcn_fdot2(a1, as_h2(pw[h]), o[h][k][1], false);
                }
            }
        }
    };
    // one 64-token tile: blocks s0 and s0 + 32 (A holds the first, already
    // loaded, when the next tile's first block is prefetched).
    //  - d <= 128: each block's K runs through the MFMAs and its V into its
    //    32 rows of the 64-row LDS tile; the next tile's first block is
    //    loaded into A as soon as A is used (holding it doubles the load
    //    registers; measured, it pays even where it leaves one wave per SIMD,
    //    8 pieces per half row: fp16 at d = 128).
    //  - d = 256 (kSplitV): both blocks' K run through the MFMAs, then each
    //    block's V goes through one 32-row LDS tile in turn.  Halving the LDS
    //    tile and the load registers lets two wavefronts share a SIMD: the
    //    Gemma-shaped call went from 42% to 48.6% of the HBM peak, while at
    //    d = 128 this order was 1-3% slower than the one above.  Both blocks
    //    are loaded at the tile's start: loading the next tile's K and V
    //    into the same registers as soon as this tile's are consumed keeps
    //    them live through the softmax and p.V, and needed more registers
    //    than two wavefronts per SIMD leave (spills at every tier).
    // (The prefetch is a compile-time choice: a load issued on one branch
    // only would make the wait counts of the merged paths conservative.)
    constexpr bool PREF = !kSplitV && NPH <= 8;
    auto tile_body = [&](auto masked, auto prefetch, int64_t s0) {
        constexpr bool MASKED = decltype(masked)::value;
        constexpr bool PREFETCH = PREF && decltype(prefetch)::value;
        f16v c[2];
        if constexpr (kSplitV) {
            load_block(A, s0);
            load_block(B, s0 + 32);
            k_block(A, c[0]);
            k_block(B, c[1]);
        } else {
            if constexpr (!PREF) load_block(A, s0);
            load_block(B, s0 + 32);
            if constexpr (PREF) pin(A);
            k_block(A, c[0]);
            v_block(A, 0);
            if constexpr (PREFETCH) load_block(A, s0 + 64);
            if constexpr (PREF) pin(B);
            k_block(B, c[1]);
            v_block(B, 32);
        }

        // S^T fragment: lane holds head r, tokens 32*blk + 8*(e/4) + 4*hb + e%4
        if constexpr (MASKED) {
            const int rem = (int)(N - s0);
#pragma unroll
            for (int blk = 0; blk < 2; ++blk)
#pragma unroll
                for (int e = 0; e < 16; ++e)
                    if (32 * blk + 8 * (e / 4) + 4 * hb + (e % 4) >= rem) c[blk][e] = -INFINITY;
        }
        float mx = -INFINITY;
#pragma unroll
        for (int blk = 0; blk < 2; ++blk)
#pragma unroll
            for (int e = 0; e < 16; ++e) mx = fmaxf(mx, c[blk][e]);
        mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
        const float mn = fmaxf(m, mx * a.c2);
        const float alpha = __builtin_amdgcn_exp2f(m - mn);  // 0 on the first tile
        m = mn;
        const h2 ones = {(_Float16)1.0f, (_Float16)1.0f};
        float ps = 0.0f;
#pragma unroll
        for (int blk = 0; blk < 2; ++blk)
#pragma unroll
            for (int e = 0; e < 16; e += 4) {
                h2 p01, p23;
                p01.x = (_Float16)__builtin_amdgcn_exp2f(fmaf(c[blk][e], a.c2, -mn));
                p01.y = (_Float16)__builtin_amdgcn_exp2f(fmaf(c[blk][e + 1], a.c2, -mn));
                p23.x = (_Float16)__builtin_amdgcn_exp2f(fmaf(c[blk][e + 2], a.c2, -mn));
                p23.y = (_Float16)__builtin_amdgcn_exp2f(fmaf(c[blk][e + 3], a.c2, -mn));
                ps = __builtin_amdgcn_fdot2(p01, ones, ps, false);
                ps = __builtin_amdgcn_fdot2(p23, ones, ps, false);
                if (r < GM) {
                    // token pairs (32*blk + 8*(e/4) + 4*hb) / 2 and the next one
                    const int pi = 16 * blk + 4 * (e / 4) + 2 * hb;
                    pp[pi * GM + r] = as_u32(p01);
                    pp[(pi + 1) * GM + r] = as_u32(p23);
                }
            }
        lsum = lsum * alpha + ps;
#pragma unroll
        for (int h = 0; h < GM; ++h) {
            const float al = __shfl(alpha, h, 64);
#pragma unroll
            for (int k = 0; k < DWL; ++k) {
                o[h][k][0] *= al;
                o[h][k][1] *= al;
            }
        }
        using p16 = std::integral_constant<int, 16>;
        using p32 = std::integral_constant<int, 32>;
        if constexpr (kSplitV) {
            v_block(A, 0);
            __syncthreads();
            pv_rows(p16{}, 0, 0);
            __syncthreads();
            v_block(B, 0);
            __syncthreads();
            pv_rows(p16{}, 16, 0);
        } else {
            __syncthreads();
            pv_rows(p32{}, 0, 0);
        }
        __syncthreads();
    };

    using yes = std::integral_constant<bool, true>;
    using no = std::integral_constant<bool, false>;
    const int64_t c0 = chunk * a.T * 64;
    const int64_t c1 = c0 + a.T * 64 < N ? c0 + a.T * 64 : N;  // end of this chunk
    const int64_t nfull = (c1 - c0) / 64;                       // whole tiles
    const bool tail = c0 + nfull * 64 < c1;
    if constexpr (PREF) load_block(A, c0);
    int64_t s0 = c0;
    for (int64_t t = 0; t + 1 < nfull; ++t, s0 += 64) tile_body(no{}, yes{}, s0);
    if (nfull > 0) {
        if (tail)
            tile_body(no{}, yes{}, s0);
        else
            tile_body(no{}, no{}, s0);
        s0 += 64;
    }
    if (tail) tile_body(yes{}, no{}, s0);

    // lanes r and r + 32 hold the same head's two token halves
    const float ltot = lsum + __shfl_xor(lsum, 32, 64);
    float* recs = a.part + (((int64_t)li * a.Hq + (int64_t)g * G) * a.NC + ta.chunk_base + chunk) *
                               (D + 2);
    const int64_t hstride = a.NC * (D + 2);  // between consecutive heads
    if (lane < G) {
        recs[lane * hstride] = m;
        recs[lane * hstride + 1] = ltot;
    }
#pragma unroll
    for (int h = 0; h < GM; ++h) {
        if constexpr (TG > 1) {
#pragma unroll
            for (int k = 0; k < DWL; ++k) {
                o[h][k][0] += __shfl_xor(o[h][k][0], 32, 64);
                o[h][k][1] += __shfl_xor(o[h][k][1], 32, 64);
            }
        }
        if (h >= G) continue;
        if (lane < LPT) {
            float* rec = recs + h * hstride;
#pragma unroll
            for (int k = 0; k < DWL; ++k) {
                const int c = pair_channel<TIER>(lane + k * LPT);
                rec[2 + c] = o[h][k][0];
                rec[2 + c + pair_step<TIER>()] = o[h][k][1];
            }
        }
    }
}

// Decode attention with both contractions on the matrix cores, on
// v_mfma_f32_16x16x32_f16 (per 64-lane wavefront: A holds row l%16 with
// k = 8*(l/16) .. +7, B holds column l%16 with the same k, and D[4*(l/16)+i]
// [l%16] sits in lane l).  Lane l works on column c = l%16 and lane group
// q = l/16:
//   - S^T = K Q^T per 16-token tile: A = K (row = token c of the tile, its
//     quarter q of the dims, d/32 MFMAs), B = Q^T (column = head c of the
//     group, zero past G), so lane l ends with the scores of head c for the
//     tokens 4q .. 4q+3 of the tile;
//   - softmax per head: the lane's 16 scores of a 64-token tile, then a max
//     over the four lanes of its head (l, l^16, l^32, l^48);
//   - O^T = V^T P^T per 32-token block: B = P^T is exactly the lane's own
//     probabilities (k = 8q + j: token 4q + j of the block's first tile for
//     j < 4, token 16 + 4q + j - 4 of its second), A = V^T comes from the
//     token-major V rows in LDS through ds_read_b64_tr_b16, which hands lane
//     j of a 16-lane group element j%4 of the 8-byte read of lane 4r+j/4,
//     r = 0..3: with lane 4r+s reading token T0+r, channels c0+4s .. +3,
//     lane j gets channel c0+j of tokens T0 .. T0+3, the same k order;
//     D is O^T: lane l holds channels 16t + 4q + i of head c, so the online
//     softmax rescale stays in the lane.
// Against the VALU form above this takes the p.V dot products (about a
// quarter of the VALU instructions) and half the exponentials (16 instead of
// 32 per lane and tile: a 16-column tile wastes less on a small query group)
// off the vector ALUs.  The dequantized values, the fp16 probabilities and
// the fp32 accumulation are the same.
typedef float f4v __attribute__((ext_vector_type(4)));
typedef short v4s __attribute__((ext_vector_type(4)));

template <int D>
constexpr int mfma_vt_pitch() { return D + 16; }  // halfs: 2D + 32 bytes, so the
                                                  // 8 rows of a half-wave's
                                                  // transposing reads hit 8
                                                  // disjoint bank groups

// Channel held at position p of a dequantized row (int4 rows come in deq4's
// pair order: positions 2m, 2m+1 of each group of 8 hold channels m, m + 4).
template <int TIER>
__device__ __forceinline__ int pos_channel(int p) {
    return TIER == 2 ? (p & ~7) + ((p >> 1) & 3) + 4 * (p & 1) : p;
}

template <int NPQ>
struct QuarterRegs {
    u32x4 k[2][NPQ], v[2][NPQ];  // [16-token tile][16-byte piece]
    uint16_t sk[2], sv[2];
};

// LDS of one wavefront of the matrix-core body: its V rows, then (P4) the
// probability table.
template <int D, int TIER, bool P4>
constexpr bool half_v() { return P4 && D == 256 && TIER == 2; }

template <int D>
constexpr size_t mfma_wave_lds() { return (size_t)32 * mfma_vt_pitch<D>() * 2 + 4 * 64 * 2; }

// Ordering of one wavefront's own LDS writes and reads.  The wavefront
// issues its LDS instructions in order, so only the compiler's code motion
// has to be stopped; with several wavefronts per workgroup, each on LDS of
// its own, a workgroup barrier would only make them wait for each other.
template <bool WG>
__device__ __forceinline__ void lds_sync() {
    if constexpr (WG) {
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
        __builtin_amdgcn_wave_barrier();
    } else {
        __syncthreads();
    }
}

template <int D, int TIER, bool P4, bool WG>
__device__ __forceinline__ void partial_mfma(const PartialArgs& a, const TierArgs& ta,
                                             int64_t chunk, int g, _Float16* vt, _Float16* pt) {
    using TI = Tier<D, TIER>;
    constexpr int DQ = D / 4;            // dims of a quarter row
    constexpr int QBYTES = TI::RB / 4;   // its bytes
    constexpr int NPQ = QBYTES / 16;     // its 16-byte pieces
    constexpr int PPP = TI::PPP;         // fp16 pairs per piece
    constexpr int KC = D / 32;           // MFMAs per S^T tile
    constexpr int CT = D / 16;           // channel tiles of O^T
    constexpr int PV = mfma_vt_pitch<D>();
    static_assert(NPQ >= 1 && NPQ * PPP / 4 == KC, "a quarter row feeds the S^T MFMAs");

    const int lane = threadIdx.x & 63;
    const int c = lane & 15;   // token of a tile (K, V), head (Q, S, P, O), channel (V^T)
    const int q = lane >> 4;   // lane group
    const int li = blockIdx.z;
    const int64_t layer = a.layer0 + li;
    const int G = a.G;
    const int64_t N = ta.N;

    // Q^T as the B operand of S^T: column c = head g*G + c (zero past G), k =
    // dims DQ*q + 8*kc .. +7
    h8 qb[KC];
    {
        const uint32_t* qrow = reinterpret_cast<const uint32_t*>(a.q) +
                               ((int64_t)li * a.Hq + (int64_t)g * G + (c < G ? c : 0)) * (D / 2) +
                               q * (DQ / 2);
#pragma unroll
        for (int kc = 0; kc < KC; ++kc) {
            u32x4 v = *reinterpret_cast<const u32x4*>(qrow + 4 * kc);
            if (c >= G) v = u32x4{0u, 0u, 0u, 0u};
            if constexpr (TIER == 2) {
                v = u32x4{__builtin_amdgcn_perm(v.z, v.x, 0x05040100u),
                          __builtin_amdgcn_perm(v.z, v.x, 0x07060302u),
                          __builtin_amdgcn_perm(v.w, v.y, 0x05040100u),
                          __builtin_amdgcn_perm(v.w, v.y, 0x07060302u)};
            }
            qb[kc] = __builtin_bit_cast(h8, v);
        }
    }

    // Loads of the 32-token block `blk` of the tile at slot s0: quarter q of
    // the K and V rows of tokens s0 + 32 blk + c and s0 + 32 blk + 16 + c.
    // Slots past the tier's end re-load its last token (they are masked);
    // only the last, partial tile has such slots.
    //
    // At d = 256 the loads are buffer loads: a tile's rows lie in one span of at
    // most 64 tokens x 2H rows (under 2^32 bytes for the at most 65535 KV heads
    // a decode call admits), so each goes through a resource at the tile's first
    // token (wave-uniform, formed with scalar arithmetic once per tile, its
    // range ending at the last byte of the tile's last token) with one 32-bit
    // per-lane offset per row that stays the same from tile to tile, and the
    // wave-uniform rest (piece, V after K) in the scalar offset operand; every
    // offset lies in the range by construction (the hardware checks only the
    // per-lane part).  That takes the 64-bit address arithmetic, the slot clamp
    // and the quarter-rate multiplies off the VALU, which the int4
    // dequantization keeps busy there: 2-3% faster on the Gemma-shaped call,
    // same outputs.  At d = 128 the same form measured 2% slower on the Qwen-
    // shaped call, so the flat form with a clamped slot per row stays.
    const uint8_t* code = a.payload + ta.off_code + q * QBYTES;
    const uint16_t* scale = reinterpret_cast<const uint16_t*>(a.payload + ta.off_scale);
    auto load_block_flat = [&](QuarterRegs<NPQ>& R, int64_t b0) {
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const int64_t slot = b0 + 16 * t + c < N ? b0 + 16 * t + c : N - 1;
            const int64_t rowK = ((layer * N + slot) * 2) * a.H + g;
            const int64_t rowV = rowK + a.H;
#pragma unroll
            for (int i = 0; i < NPQ; ++i) {
                R.k[t][i] = ld16(code + rowK * TI::RB + i * 16);
                R.v[t][i] = ld16(code + rowV * TI::RB + i * 16);
            }
            if constexpr (TIER != 0) {
                R.sk[t] = scale[rowK];
                R.sv[t] = scale[rowV];
            }
        }
    };
    const int64_t rows_tok = 2 * (int64_t)a.H;  // K and V rows of a token
    const uint8_t* code_l = a.payload + ta.off_code + layer * N * rows_tok * TI::RB;
    const uint8_t* scale_l = a.payload + ta.off_scale + layer * N * rows_tok * 2;
    const uint32_t vcode = (uint32_t)a.H * TI::RB;  // a token's V row after its K row
    const uint32_t vscale = (uint32_t)a.H * 2;
    // byte offsets of quarter q of head g's K row (code, scale) of the token
    // `rel` slots after a tile's first
    auto lane_off = [&](int64_t rel, uint32_t& oc, uint32_t& os) {
        oc = (uint32_t)((rel * rows_tok + g) * TI::RB + q * QBYTES);
        os = (uint32_t)((rel * rows_tok + g) * 2);
    };
    uint32_t ocode[4], oscale[4];  // tokens 16u + c of a tile, u = 0..3
#pragma unroll
    for (int u = 0; u < 4; ++u) lane_off(16 * u + c, ocode[u], oscale[u]);
    auto load_block = [&](QuarterRegs<NPQ>& R, int64_t s0, int blk, auto masked) {
        if constexpr (D != 256) {
            load_block_flat(R, s0 + 32 * blk);
        } else {
            const int64_t ntok = N - s0 < 64 ? N - s0 : 64;
            const __amdgpu_buffer_rsrc_t rc =
                make_rsrc(code_l + s0 * rows_tok * TI::RB, (uint32_t)(ntok * rows_tok * TI::RB));
            const __amdgpu_buffer_rsrc_t rs =
                make_rsrc(scale_l + s0 * rows_tok * 2, (uint32_t)(ntok * rows_tok * 2));
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                uint32_t oc = ocode[2 * blk + t], os = oscale[2 * blk + t];
                if constexpr (decltype(masked)::value) {
                    const int64_t rel = 32 * blk + 16 * t + c;
                    lane_off(rel < ntok ? rel : ntok - 1, oc, os);
                }
#pragma unroll
                for (int i = 0; i < NPQ; ++i) {
                    R.k[t][i] = __builtin_bit_cast(
                        u32x4, __builtin_amdgcn_raw_buffer_load_b128(rc, oc, i * 16, 0));
                    R.v[t][i] = __builtin_bit_cast(
                        u32x4, __builtin_amdgcn_raw_buffer_load_b128(rc, oc, vcode + i * 16, 0));
                }
                if constexpr (TIER != 0) {
                    R.sk[t] = __builtin_amdgcn_raw_buffer_load_b16(rs, os, 0, 0);
                    R.sv[t] = __builtin_amdgcn_raw_buffer_load_b16(rs, os, vscale, 0);
                }
            }
        }
    };
    auto scale2 = [&](uint16_t bits) -> h2 {
        if constexpr (TIER == 0) {
            return h2{(_Float16)1.0f, (_Float16)1.0f};
        } else {
            uint32_t sb = bits;
            asm volatile("" : "+v"(sb));  // consumed here, not where it was loaded
            return as_h2(sb | (sb << 16));
        }
    };
    // S^T of the block's two 16-token tiles
    auto s_block = [&](const QuarterRegs<NPQ>& R, f4v (&st)[2]) {
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const h2 sk2 = scale2(R.sk[t]);
            f4v acc = f4v{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int i = 0; i < NPQ; ++i) {
                uint32_t pr[PPP];
                piece_pairs<D, TIER>(R.k[t][i], sk2, pr);
#pragma unroll
                for (int j = 0; j < PPP / 4; ++j)
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                        pairs_h8(pr[4 * j], pr[4 * j + 1], pr[4 * j + 2], pr[4 * j + 3]),
                        qb[i * (PPP / 4) + j], acc, 0, 0, 0);
            }
            st[t] = acc;
        }
    };
    // the block's dequantized V rows into LDS (row = token of the block)
    // (tiles t0 .. t1 - 1 of the block, tile t at rows 16 * (t - t0) ..)
    auto v_block = [&](const QuarterRegs<NPQ>& R, int t0, int t1) {
#pragma unroll
        for (int t = t0; t < t1; ++t) {
            const h2 sv2 = scale2(R.sv[t]);
            _Float16* vrow = vt + (16 * (t - t0) + c) * PV + DQ * q;
#pragma unroll
            for (int i = 0; i < NPQ; ++i) {
                uint32_t pv[PPP];
                piece_pairs<D, TIER>(R.v[t][i], sv2, pv);
#pragma unroll
                for (int e = 0; e < PPP; e += 4)
                    *reinterpret_cast<u32x4*>(vrow + 2 * (i * PPP + e)) =
                        u32x4{pv[e], pv[e + 1], pv[e + 2], pv[e + 3]};
            }
        }
    };

    float m = -INFINITY, lsum = 0.0f;  // head c, base-2 domain; lsum over this lane's tokens
    // O^T accumulators: CT 16x16 tiles, or with P4 (G <= 4) D/64 groups of
    // the 4x4x4 form, whose lane l holds channels 64*mg + 4*(l/4) + i of head
    // l%4
    constexpr int NO = P4 ? D / 64 : CT;
    // int4 rows at d = 256 stage V 16 tokens at a time in the 4x4x4 form:
    // 8.7 KB of LDS per wavefront instead of 17, so the three wavefronts per
    // SIMD that its registers allow fit (538 against 561-570 us on the
    // Gemma-shaped int4 tier; int8, at two wavefronts either way, lost 15%).
    constexpr bool HALF_V = half_v<D, TIER, P4>();
    f4v o[NO];
#pragma unroll
    for (int t = 0; t < NO; ++t) o[t] = f4v{0.0f, 0.0f, 0.0f, 0.0f};
    // this lane's transposing-read address: token 4q + c/4, channels 4*(c%4) ..
    // (with P4: token c/4, channels 16q + 4*(c%4) .., 64 channels per group)
    _Float16* vrd = P4 ? vt + (c >> 2) * PV + 16 * q + 4 * (c & 3)
                       : vt + (4 * q + (c >> 2)) * PV + 4 * (c & 3);

    QuarterRegs<NPQ> A, B;
    auto tile_body = [&](auto masked, int64_t s0) {
        constexpr bool MASKED = decltype(masked)::value;
        load_block(A, s0, 0, masked);
        load_block(B, s0, 1, masked);
        f4v st[2][2];
        s_block(A, st[0]);
        s_block(B, st[1]);
        // lane: head c, tokens 32*blk + 16*t + 4*q + i of the tile
        if constexpr (MASKED) {
            const int rem = (int)(N - s0);
#pragma unroll
            for (int blk = 0; blk < 2; ++blk)
#pragma unroll
                for (int t = 0; t < 2; ++t)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        if (32 * blk + 16 * t + 4 * q + i >= rem) st[blk][t][i] = -INFINITY;
        }
        float mx = -INFINITY;
#pragma unroll
        for (int blk = 0; blk < 2; ++blk)
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int i = 0; i < 4; ++i) mx = fmaxf(mx, st[blk][t][i]);
        mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
        mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
        const float mn = fmaxf(m, mx * a.c2);
        const float alpha = __builtin_amdgcn_exp2f(m - mn);  // 0 on the first tile
        m = mn;
        // probabilities, rounded to fp16 once: the B operand of each block's
        // O^T MFMAs and the terms of the denominator
        h8 pb[2];
        float ps = 0.0f;
        const h2 ones = {(_Float16)1.0f, (_Float16)1.0f};
#pragma unroll
        for (int blk = 0; blk < 2; ++blk) {
            uint32_t pw[4];
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int i = 0; i < 4; i += 2) {
                    h2 pr;
                    pr.x = (_Float16)__builtin_amdgcn_exp2f(fmaf(st[blk][t][i], a.c2, -mn));
                    pr.y = (_Float16)__builtin_amdgcn_exp2f(fmaf(st[blk][t][i + 1], a.c2, -mn));
                    ps = __builtin_amdgcn_fdot2(pr, ones, ps, false);
                    pw[2 * t + i / 2] = as_u32(pr);
                }
            pb[blk] = pairs_h8(pw[0], pw[1], pw[2], pw[3]);
        }
        lsum = lsum * alpha + ps;
        if constexpr (P4) {
            // this tile's probabilities of heads 0..3 by token, for the B
            // operand of the 4x4x4 form (lane l reads head l%4)
            if (c < 4) {
#pragma unroll
                for (int blk = 0; blk < 2; ++blk)
#pragma unroll
                    for (int t = 0; t < 2; ++t)
                        *reinterpret_cast<uint2*>(pt + c * 64 + 32 * blk + 16 * t + 4 * q) =
                            make_uint2(__builtin_bit_cast(u32x4, pb[blk])[2 * t],
                                       __builtin_bit_cast(u32x4, pb[blk])[2 * t + 1]);
            }
            const float al = __shfl(alpha, lane & 3, 64);
            if (!__all(al == 1.0f)) {
#pragma unroll
                for (int t = 0; t < NO; ++t) o[t] *= al;
            }
        } else if (!__all(alpha == 1.0f)) {
#pragma unroll
            for (int t = 0; t < CT; ++t) o[t] *= alpha;
        }
        typedef __attribute__((address_space(3))) v4s lds_v4s;
#pragma unroll
        for (int blk = 0; blk < 2; ++blk) {
            if constexpr (P4) {
                // 4x4x4 form, 16 blocks per instruction: block b = l/4 holds
                // channels 64*mg + 4b .. +3 (rows, A from the transposing
                // read: lane 4b + i gets channel 64*mg + 4b + i of 4 tokens)
                // by heads 0..3 (columns, B: lane 4b + j gets head j's 4
                // probabilities), k = 4 tokens per step; with HALF_V the
                // block's V goes through LDS one 16-token tile at a time
#pragma unroll
                for (int h = 0; h < (HALF_V ? 2 : 1); ++h) {
                    v_block(blk == 0 ? A : B, HALF_V ? h : 0, HALF_V ? h + 1 : 2);
                    lds_sync<WG>();
#pragma unroll
                    for (int kk = 0; kk < (HALF_V ? 4 : 8); ++kk) {
                        const h4 pj = *reinterpret_cast<const h4*>(
                            pt + (lane & 3) * 64 + 32 * blk + 16 * h + 4 * kk);
#pragma unroll
                        for (int mg = 0; mg < NO; ++mg) {
                            const v4s va = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                                (lds_v4s*)(vrd + 4 * kk * PV + 64 * mg));
                            o[mg] = __builtin_amdgcn_mfma_f32_4x4x4f16(
                                __builtin_bit_cast(h4, va), pj, o[mg], 0, 0, 0);
                        }
                    }
                    if (HALF_V && h == 0) lds_sync<WG>();
                }
            } else {
                v_block(blk == 0 ? A : B, 0, 2);
                lds_sync<WG>();
#pragma unroll
                for (int t = 0; t < CT; ++t) {
                    const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (lds_v4s*)(vrd + 16 * t));
                    const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (lds_v4s*)(vrd + 16 * PV + 16 * t));
                    const h8 va = __builtin_shufflevector(__builtin_bit_cast(h4, lo),
                                                          __builtin_bit_cast(h4, hi), 0, 1, 2,
                                                          3, 4, 5, 6, 7);
                    o[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(va, pb[blk], o[t], 0, 0, 0);
                }
            }
            lds_sync<WG>();
        }
    };

    using yes = std::integral_constant<bool, true>;
    using no = std::integral_constant<bool, false>;
    const int64_t c0 = chunk * a.T * 64;
    const int64_t c1 = c0 + a.T * 64 < N ? c0 + a.T * 64 : N;  // end of this chunk
    const int64_t nfull = (c1 - c0) / 64;                       // whole tiles
    int64_t s0 = c0;
    for (int64_t t = 0; t < nfull; ++t, s0 += 64) tile_body(no{}, s0);
    if (s0 < c1) tile_body(yes{}, s0);

    // the four lanes of a head hold disjoint tokens' sums
    float ltot = lsum + __shfl_xor(lsum, 16, 64);
    ltot += __shfl_xor(ltot, 32, 64);
    const int64_t rec0 = (int64_t)li * a.Hq + (int64_t)g * G;  // record row of head 0
    const int64_t rstride = a.NC * (D + 2);                      // between heads
    float* rec = a.part + (rec0 * a.NC + ta.chunk_base + chunk) * (D + 2);
    if (c < G && q == 0) {
        rec[c * rstride] = m;
        rec[c * rstride + 1] = ltot;
    }
    if constexpr (P4) {
        const int j = lane & 3;  // head
        if (j < G) {
#pragma unroll
            for (int mg = 0; mg < NO; ++mg)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    rec[j * rstride + 2 + pos_channel<TIER>(64 * mg + 4 * (lane >> 2) + i)] =
                        o[mg][i];
        }
    } else if (c < G) {
#pragma unroll
        for (int t = 0; t < CT; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                rec[c * rstride + 2 + pos_channel<TIER>(16 * t + 4 * q + i)] = o[t][i];
    }
}

// The matrix-core body covers d = 128 and 256 except fp16 rows at d = 256,
// whose two blocks of quarter rows would need 256 load registers.
template <int D, int TIER>
constexpr bool use_mfma_body() { return D >= 128 && !(D == 256 && TIER == 0); }

template <int D, int TIER, bool P4>
__global__ __launch_bounds__(64) void decode_mfma_kernel(PartialArgs a) {
    __shared__ __align__(16) _Float16 vt[(half_v<D, TIER, P4>() ? 16 : 32) * mfma_vt_pitch<D>()];
    __shared__ __align__(16) _Float16 pt[P4 ? 4 * 64 : 4];
    partial_mfma<D, TIER, P4, false>(a, a.tier[TIER], blockIdx.x, blockIdx.y, vt, pt);
}

// The fp16 and int4 tiers in one launch when both are a few chunks (sinks
// and a handful of int4 tokens at b = 0.5): blocks below the fp16 tier's
// chunk count run that tier, the others the int4 tier.  At d = 128 both
// use the matrix-core body with the same LDS; one launch instead of two
// saves the second launch's fill and drain (about 5 us).
constexpr int64_t kTinyChunks = 4;

template <int D, bool P4>
__global__ __launch_bounds__(64) void decode_mfma_tiny_kernel(PartialArgs a, int chunks0) {
    static_assert(!half_v<D, 0, P4>() && !half_v<D, 2, P4>(), "same LDS for both tiers");
    __shared__ __align__(16) _Float16 vt[32 * mfma_vt_pitch<D>()];
    __shared__ __align__(16) _Float16 pt[P4 ? 4 * 64 : 4];
    if ((int)blockIdx.x < chunks0)
        partial_mfma<D, 0, P4, false>(a, a.tier[0], blockIdx.x, blockIdx.y, vt, pt);
    else
        partial_mfma<D, 2, P4, false>(a, a.tier[2], blockIdx.x - chunks0, blockIdx.y, vt, pt);
}

// KV heads (wavefronts) of a workgroup of the one-per-head form: eight keep
// the register budget of two wavefronts per SIMD.
constexpr int kWgMaxHeads = 8;
// Workgroups a launch needs before the one-per-head form is used: two per CU.
constexpr int64_t kWgMinGroups = 512;

// One workgroup per (layer, tier, chunk) with one wavefront per KV head:
// the token rows of a chunk hold every head's K (then V) row side by side,
// so the wavefronts of a workgroup read them as one contiguous stream
// instead of one row in 2H per wavefront.
template <int D, int TIER, bool P4>
__global__ __launch_bounds__(64 * kWgMaxHeads) void decode_mfma_wg_kernel(PartialArgs a) {
    extern __shared__ __align__(16) _Float16 lds[];
    const int w = threadIdx.x >> 6;
    _Float16* vt = lds + w * (mfma_wave_lds<D>() / 2);
    _Float16* pt = vt + 32 * mfma_vt_pitch<D>();
    partial_mfma<D, TIER, P4, true>(a, a.tier[TIER], blockIdx.x, w, vt, pt);
}

// One launch per tier (a single kernel holding all three bodies would need
// registers for their union): blockIdx.x is the chunk within the tier.
template <int D, int TIER, int GM>
__global__ __launch_bounds__(64) void decode_partial_kernel(PartialArgs a) {
    __shared__ uint32_t vt[(D == 256 ? 32 : 64) * lds_pitch<D>()];
    __shared__ uint32_t pp[32 * GM];
    partial_body<D, TIER, GM>(a, a.tier[TIER], blockIdx.x, vt, pp);
}

// One wavefront per (layer, query head): chunks combined in index order.
template <int D>
__global__ __launch_bounds__(64) void merge_kernel(const float* __restrict__ part, int64_t NC,
                                                   int Hq, float* __restrict__ out,
                                                   float* __restrict__ lse) {
    constexpr int CPL = (D + 63) / 64;  // channels per lane
    // chunks whose loads are in flight together: with 16, the 65 chunk
    // records of a Qwen- or Gemma-shaped (layer, head) take 5 round trips to
    // memory instead of 17 (12.0 -> 9.8 us at d = 128, 20.8 -> 16.5 us at
    // d = 256); the additions keep chunk order, so the result is unchanged
    constexpr int U = 16;
    const int lane = threadIdx.x;
    const int h = blockIdx.x;
    const int li = blockIdx.y;
    const float* rec0 = part + ((int64_t)li * Hq + h) * NC * (D + 2);
    float M = -INFINITY;
    for (int64_t c = lane; c < NC; c += 64) M = fmaxf(M, rec0[c * (D + 2)]);
    M = wave_max(M);
    float L = 0.0f, acc[CPL];
#pragma unroll
    for (int k = 0; k < CPL; ++k) acc[k] = 0.0f;
    if (M != -INFINITY) {
        for (int64_t c0 = 0; c0 < NC; c0 += U) {
            float w[U], l[U], v[U][CPL];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int64_t c = c0 + u < NC ? c0 + u : NC - 1;
                const float* rec = rec0 + c * (D + 2);
                w[u] = c0 + u < NC ? rec[0] : -INFINITY;
                l[u] = rec[1];
#pragma unroll
                for (int k = 0; k < CPL; ++k) {
                    const int ch = lane + 64 * k;
                    v[u][k] = ch < D ? rec[2 + ch] : 0.0f;
                }
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const float e = __builtin_amdgcn_exp2f(w[u] - M);  // 0 for an empty chunk
                L += e * l[u];
#pragma unroll
                for (int k = 0; k < CPL; ++k) acc[k] += e * v[u][k];
            }
        }
    }
    float* o = out + ((int64_t)li * Hq + h) * D;
#pragma unroll
    for (int k = 0; k < CPL; ++k) {
        const int ch = lane + 64 * k;
        if (ch < D) o[ch] = L > 0.0f ? acc[k] / L : 0.0f;
    }
    if (lse && lane == 0)
        lse[(int64_t)li * Hq + h] = L > 0.0f ? (M + log2f(L)) * 0.69314718055994531f : -INFINITY;
}

// LDS a workgroup may take on the current device (read once per device).
size_t wg_lds_limit() {
    static std::atomic<int> cached[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
    int v = cached[dev].load(std::memory_order_relaxed);
    if (v == 0) {
        if (hipDeviceGetAttribute(&v, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) !=
                hipSuccess ||
            v <= 0)
            return 0;
        cached[dev].store(v, std::memory_order_relaxed);
    }
    return (size_t)v;
}

template <int D, int TIER>
hipError_t launch_tier(const PartialArgs& a, int nl, int GM, hipStream_t st) {
    const int64_t chunks = a.cend[TIER] - a.tier[TIER].chunk_base;
    if (chunks == 0) return hipSuccess;
    const dim3 grid((unsigned)chunks, (unsigned)a.H, (unsigned)nl);
    if constexpr (use_mfma_body<D, TIER>()) {
        // The one-per-head workgroups pay at d = 128 when they are enough
        // to fill the machine twice over (measured: Mistral-shaped int8 tier,
        // 512 workgroups, 128 -> 110 us).  With fewer, or at d = 256, where
        // a workgroup takes most of a CU's LDS, they were 3-36% slower than
        // one wavefront per workgroup.
        const size_t wg_lds = (size_t)a.H * mfma_wave_lds<D>();
        if (D == 128 && a.H <= kWgMaxHeads && chunks * nl >= kWgMinGroups &&
            wg_lds <= wg_lds_limit()) {
            if constexpr (D == 128) {
                const dim3 wgrid((unsigned)chunks, 1u, (unsigned)nl);
                if (GM <= 4)
                    decode_mfma_wg_kernel<D, TIER, true><<<wgrid, 64 * a.H, wg_lds, st>>>(a);
                else
                    decode_mfma_wg_kernel<D, TIER, false><<<wgrid, 64 * a.H, wg_lds, st>>>(a);
                return hipGetLastError();
            }
        }
        if (GM <= 4)
            decode_mfma_kernel<D, TIER, true><<<grid, 64, 0, st>>>(a);
        else
            decode_mfma_kernel<D, TIER, false><<<grid, 64, 0, st>>>(a);
    } else {
        switch (GM) {
            case 1: decode_partial_kernel<D, TIER, 1><<<grid, 64, 0, st>>>(a); break;
            case 2: decode_partial_kernel<D, TIER, 2><<<grid, 64, 0, st>>>(a); break;
            case 4: decode_partial_kernel<D, TIER, 4><<<grid, 64, 0, st>>>(a); break;
            case 8: decode_partial_kernel<D, TIER, 8><<<grid, 64, 0, st>>>(a); break;
            default: decode_partial_kernel<D, TIER, 16><<<grid, 64, 0, st>>>(a); break;
        }
    }
    return hipGetLastError();
}

template <int D>
hipError_t launch_all(const PartialArgs& a, int nl, int GM, float* out, float* lse,
                      hipStream_t st) {
    hipError_t e = launch_tier<D, 1>(a, nl, GM, st);
    const int64_t ch0 = a.cend[0] - a.tier[0].chunk_base;
    const int64_t ch2 = a.cend[2] - a.tier[2].chunk_base;
    bool tiny = false;
    if constexpr (D == 128) tiny = ch0 > 0 && ch2 > 0 && ch0 + ch2 <= kTinyChunks;
    if (tiny) {
        if constexpr (D == 128) {
            const dim3 grid((unsigned)(ch0 + ch2), (unsigned)a.H, (unsigned)nl);
            if (e == hipSuccess) {
                if (GM <= 4)
                    decode_mfma_tiny_kernel<D, true><<<grid, 64, 0, st>>>(a, (int)ch0);
                else
                    decode_mfma_tiny_kernel<D, false><<<grid, 64, 0, st>>>(a, (int)ch0);
                e = hipGetLastError();
            }
        }
    } else {
        if (e == hipSuccess) e = launch_tier<D, 2>(a, nl, GM, st);
        if (e == hipSuccess) e = launch_tier<D, 0>(a, nl, GM, st);
    }
    if (e != hipSuccess) return e;
    merge_kernel<D><<<dim3((unsigned)a.Hq, (unsigned)nl), 64, 0, st>>>(a.part, a.NC, a.Hq, out,
                                                                      lse);
    return hipGetLastError();
}

}  // namespace

int decode_tiles_per_chunk(const Dims& s, const TierSeg seg[3], int nl) {
    int64_t tiles = 0;
    for (int t = 0; t < 3; ++t) tiles += (seg[t].count + 63) / 64;
    tiles *= (int64_t)s.Hkv * nl;
    int T = 1;
    while (T < 8 && tiles / (2 * T) >= 4096) T *= 2;  // keep >= 4096 wavefronts
    return T;
}

int64_t decode_chunks(const Dims& s, const TierSeg seg[3], int nl) {
    const int64_t span = 64 * (int64_t)decode_tiles_per_chunk(s, seg, nl);
    int64_t nc = 0;
    for (int t = 0; t < 3; ++t) nc += (seg[t].count + span - 1) / span;
    return nc;
}

hipError_t launch_decode(const Dims& s, const TierSeg seg[3], const void* payload, int layer0,
                         int nl, const void* q, float* out, float* lse, float* part,
                         hipStream_t st) {
    PartialArgs a;
    a.payload = static_cast<const uint8_t*>(payload);
    a.T = decode_tiles_per_chunk(s, seg, nl);
    const int64_t span = 64 * (int64_t)a.T;
    int64_t cb = 0;
    for (int t = 0; t < 3; ++t) {
        a.tier[t].off_code = seg[t].off_code;
        a.tier[t].off_scale = seg[t].off_scale;
        a.tier[t].N = seg[t].count;
        a.tier[t].chunk_base = cb;
        cb += (seg[t].count + span - 1) / span;
        a.cend[t] = cb;
    }
    a.NC = cb;
    a.H = s.Hkv;
    a.G = s.Hq / s.Hkv;
    a.Hq = s.Hq;
    a.layer0 = layer0;
    a.q = static_cast<const uint16_t*>(q);
    a.part = part;
    a.c2 = 1.4426950408889634f / sqrtf((float)s.d);
    int GM = 1;
    while (GM < a.G) GM *= 2;
    switch (s.d) {
        case 64: return launch_all<64>(a, nl, GM, out, lse, st);
        case 128: return launch_all<128>(a, nl, GM, out, lse, st);
        case 256: return launch_all<256>(a, nl, GM, out, lse, st);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace sk
