// Token importance score: causal attention column sums with MFMA.
//
// SpectrumKV paper, §4.3 (I_j = A_j exp(-lambda Delta_j), here lambda = 0) and
// Algorithm 1 "score tokens"; the score is the attention a token receives,
// summed over query heads (and, across calls, layers):
//     A_j = sum_h sum_{i >= j} softmax_i(q_i . k_j / sqrt(d))_j.
//
// The softmax of row i needs the whole row before any column can be summed,
// and storing P is O(n^2), so the path is two passes over Q K^T:
//   pass 1 (rowlse): lse2[h][i] = log2 sum_{j<=i} exp(q_i . k_j / sqrt(d)),
//                    the base-2 logarithm of the causal softmax denominator;
//   pass 2 (colsum): recompute s_ij and sum 2^(c2 s_ij - lse2_i) down each
//                    column j (c2 = log2(e)/sqrt(d)), per query head; a
//                    fixed-order reduction over heads yields the layer's A_j.
// Both passes are dense fp16 contractions on v_mfma_f32_32x32x16_f16 with
// fp32 accumulation; the softmax arithmetic is fp32 in base 2.
//
// MFMA 32x32x16 operand layout (per 64-lane wavefront):
//   A (32 x 16): lane l holds row l%32, k = 8*(l/32) .. +7
//   B (16 x 32): lane l holds column l%32, k = 8*(l/32) .. +7
//   C (32 x 32): lane l holds column l%32, rows 8*(e/4) + 4*(l/32) + e%4, e = 0..15
// A and B are both "k-contiguous", which is exactly the row-major [token][d]
// layout of Q and K, so every fragment is one 16-byte read.
//
// Cost model on gfx950 (per 32x32 tile and wavefront, measured): the d/16
// MFMAs take 2d cycles of the matrix pipe; the softmax work is 16 elements
// per lane at one fma + one exp2 + one add each (~12 cycles per element
// row).  At d >= 128 the VALU work fits under the MFMA work when the two
// overlap, so both passes keep two wavefronts per SIMD, prefetch the next
// LDS stage while computing on the current one (double buffering, one
// barrier per stage) and keep per-element work to those three operations.
//
// pass 1 computes S^T = K Q^T (rows = keys, columns = queries): each lane owns
// one query and 16 of the 32 keys of a tile, so the row sums are in-lane; the
// two half-waves' partial sums are combined once at the end.  A workgroup is
// W query heads of one GQA group times QW blocks of 64 queries (one wavefront
// each), so each staged K tile is read by every wavefront.  The key stages on
// the causal diagonal are processed first with the exact online max; they fix
// a per-row reference m, and the remaining (unmasked) stages then only add
// 2^(c2 s - m): no per-element max.  A tile whose sum exceeds 2^64 (a logit
// far above the reference) is redone with the exact update, so the result
// never overflows whatever the inputs.
//
// pass 2 computes S^T = K Q^T too, with the wavefront's stationary keys as
// the A operand: each lane owns one query column (one lse2 value per tile)
// and 16 key rows of each 32-key sub-tile, whose weights add into 16
// independent per-lane accumulators across all query tiles; the 32 query
// lanes are summed once at the end.  A workgroup is one query head and KW
// wavefronts of 64 stationary keys each; the head's query tiles and their
// lse2 values stream through LDS and are read by every wavefront.
//
// Work is causal (tiles above the diagonal are skipped) and workgroups are
// launched longest-first.  In pass 1 the GQA group index runs fastest across
// the grid, so with 8 groups each of the 8 XCDs serves one group's keys from
// its own L2.
#include <hip/hip_runtime.h>

#include <mutex>
#include <type_traits>

#include "../../include/sk.h"
#include "sk_kernels.h"

// Workspace of sk_score_noalloc (lse values, then the per-head column sums):
// a device array the library owns, so that a caller that cannot allocate
// needs no workspace.  Each GPU the library runs on holds its own copy until
// the process ends.  In host code this name is only a stand-in for the
// symbol, not a device address: the address comes from hipGetSymbolAddress,
// once per device (score_scratch below), and only that address is passed to
// kernels.
static __device__ __align__(256) unsigned char scratch[SK_SCORE_SCRATCH_BYTES];

namespace sk {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

constexpr float kLog2e = 1.4426950408889634f;
// A pass-1 tile whose partial sum exceeds this goes through the exact update.
constexpr float kTileLimit = 18446744073709551616.0f;  // 2^64
constexpr int kStageKeys = 64;   // keys per pass-1 workgroup stage (32 for d = 256)
constexpr int kColKeys = 64;     // stationary keys per pass-2 wavefront
constexpr int kColWaves = 4;     // pass-2 wavefronts per workgroup

__device__ __forceinline__ floatx16 mfma32(half8 a, half8 b, floatx16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ half8 zero8() {
    half8 z;
#pragma unroll
    for (int e = 0; e < 8; ++e) z[e] = (_Float16)0.0f;
    return z;
}

__device__ __forceinline__ floatx16 zero16() {
    floatx16 z;
#pragma unroll
    for (int e = 0; e < 16; ++e) z[e] = 0.0f;
    return z;
}

// Row within a 32x32 C tile held by element e of lane l.
__device__ __forceinline__ int crow(int e, int lane) {
    return 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
}

// Buffer resource over `bytes` bytes at `base` for raw loads: the hardware
// range check returns zeros for any load at or past the end.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                             0x00020000);
}

// Cooperative staging of ROWS tokens x D halfs (contiguous per token in
// global memory, token stride `gstride` halfs) into LDS rows of D + 8 halfs
// by NT threads, through registers, so that the loads of the next stage are
// in flight while the current one is computed on.  The row pitch of D + 8
// halfs puts the 32 rows of an MFMA fragment read at distinct bank groups.
// Each thread owns the same 16-byte pieces in every stage: its first piece
// at a fixed per-thread offset, the others a uniform number of rows further
// (an immediate for the LDS store).  The stage's buffer resource covers only
// its tokens below n, and each load's whole offset is in its per-lane VGPR
// offset (the part the range check always covers), so the check zero-fills
// the ragged tail.
template <int D, int ROWS, int NT>
struct Stager {
    static constexpr int kPieces = D / 8;           // 16-byte pieces per row
    static constexpr int kRowStep = NT / kPieces;   // rows between a thread's pieces
    static constexpr int kRegs = (ROWS + kRowStep - 1) / kRowStep;
    static_assert(NT % kPieces == 0, "whole rows per thread step");
    uint4 regs[kRegs];
    uint32_t voff;  // byte offset of this thread's first piece within a stage
    int row0;       // its row within the stage
    int loff;       // its LDS offset (halfs) within a stage buffer
    __device__ __forceinline__ void init(int tid, int64_t gstride) {
        row0 = tid / kPieces;
        const int piece = tid % kPieces;
        voff = (uint32_t)((row0 * gstride + piece * 8) * 2);
        loff = row0 * (D + 8) + piece * 8;
    }
    // g points at token t0 of this head's rows; n_left = n - t0 > 0.  The
    // range ends at the last byte of the stage's last valid row of this head
    // (not at that token's stride end, which for any head but the last lies
    // inside the next head's row and, for the last, past the tensor).
    __device__ __forceinline__ void load(const _Float16* g, int64_t n_left, int64_t gstride) {
        const int64_t rows = n_left < ROWS ? n_left : ROWS;
        const __amdgpu_buffer_rsrc_t rs =
            make_rsrc(g, (uint32_t)(((rows - 1) * gstride + D) * 2));
#pragma unroll
        for (int r = 0; r < kRegs; ++r) {
            if (ROWS % kRowStep == 0 || row0 + r * kRowStep < ROWS) {
                const auto v = __builtin_amdgcn_raw_buffer_load_b128(
                    rs, voff + (uint32_t)(r * kRowStep * gstride * 2), 0, 0);
                regs[r] = *reinterpret_cast<const uint4*>(&v);
            }
        }
    }
    __device__ __forceinline__ void store(_Float16* lds) const {
#pragma unroll
        for (int r = 0; r < kRegs; ++r)
            if (ROWS % kRowStep == 0 || row0 + r * kRowStep < ROWS)
                *reinterpret_cast<uint4*>(lds + loff + r * kRowStep * (D + 8)) = regs[r];
    }
};

// Sum over the 16 elements of a C tile of 2^(c2 x - m), in four chains.
// (Each chain starts from its first term rather than 0.0f + term: the terms
// are >= 0, so the sums are the same, without an add the compiler may not
// drop under IEEE signed-zero rules.)
__device__ __forceinline__ float tile_expsum(const floatx16& a, float c2, float m) {
    float s0 = ex2(fmaf(a[0], c2, -m));
    float s1 = ex2(fmaf(a[1], c2, -m));
    float s2 = ex2(fmaf(a[2], c2, -m));
    float s3 = ex2(fmaf(a[3], c2, -m));
#pragma unroll
    for (int e = 4; e < 16; e += 4) {
        s0 += ex2(fmaf(a[e + 0], c2, -m));
        s1 += ex2(fmaf(a[e + 1], c2, -m));
        s2 += ex2(fmaf(a[e + 2], c2, -m));
        s3 += ex2(fmaf(a[e + 3], c2, -m));
    }
    return (s0 + s1) + (s2 + s3);
}

// Exact online-softmax update of one lane's (m, s) with the 16 elements of a
// pass-1 C tile (rows = keys kt0 + crow, column = query qi).  With `masked`,
// keys above the query are excluded: `lim` = qi - kt0, and row crow is kept
// while crow <= lim.
__device__ __forceinline__ void exact_update(const floatx16& a, float c2, bool masked, int lim,
                                             int lane, float& m, float& s) {
    float mx = -INFINITY;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
        const bool keep = !masked || crow(e, lane) <= lim;
        mx = fmaxf(mx, keep ? a[e] * c2 : -INFINITY);
    }
    const float mn = fmaxf(m, mx);
    if (mn == -INFINITY) return;
    float acc = (m == -INFINITY) ? 0.0f : s * ex2(m - mn);
#pragma unroll
    for (int e = 0; e < 16; ++e) {
        const bool keep = !masked || crow(e, lane) <= lim;
        acc += keep ? ex2(fmaf(a[e], c2, -mn)) : 0.0f;
    }
    s = acc;
    m = mn;
}

// Fixed-reference update of one lane's two row sums with one 32-key unit
// (two C tiles): add 2^(c2 x - m); if a tile sum leaves [0, 2^64] in any lane
// (a logit far above the reference), that lane redoes the unit exactly.
__device__ __forceinline__ void fixed_ref_update(const floatx16 (&a)[2], float c2, int lane,
                                                 float (&m)[2], float (&s)[2]) {
    const float t0 = tile_expsum(a[0], c2, m[0]);
    const float t1 = tile_expsum(a[1], c2, m[1]);
    const bool ok = (t0 <= kTileLimit) && (t1 <= kTileLimit);
    if (__builtin_expect(__all(ok), 1)) {
        s[0] += t0;
        s[1] += t1;
    } else if (ok) {
        s[0] += t0;
        s[1] += t1;
    } else {
        exact_update(a[0], c2, false, 0, lane, m[0], s[0]);
        exact_update(a[1], c2, false, 0, lane, m[1], s[1]);
    }
}

// ---------------------------------------------------------------- pass 1 --
template <int D, int W, int QW, int KS>
__global__ __launch_bounds__(W * QW * 64, D == 256 ? 1 : 2) void rowlse_kernel(
    const _Float16* __restrict__ Q, const _Float16* __restrict__ K, float* __restrict__ lse2,
    int64_t n, int Hq, int Hkv, float c2) {
    constexpr int NT = W * QW * 64;
    constexpr int C = D / 16;
    constexpr int PITCH = D + 8;
    constexpr int U = KS / 32;  // 32-key units per stage
    constexpr int SB = KS * PITCH;  // halfs per stage buffer
    // a ring of three stage buffers [3][KS][PITCH]: stage s lives in buffer
    // s % 3 and is stored at the end of stage s - 2, before that stage's
    // barrier, so during stage s the next stage's buffer is already valid
    // (its first fragments are read ahead) and the buffer written at the end
    // of stage s (that of s + 2, last read in stage s - 1) is free
    extern __shared__ _Float16 smem[];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int col = lane & 31;
    const int khalf = 8 * (lane >> 5);
    // layer blockIdx.z of an all-layer launch: Q [L][n][Hq][D], K [L][n][Hkv][D],
    // lse2 [L][Hq][n]
    Q += (int64_t)blockIdx.z * n * Hq * D;
    K += (int64_t)blockIdx.z * n * Hkv * D;
    lse2 += (int64_t)blockIdx.z * Hq * n;
    const int R = Hq / Hkv;
    const int chunks = R / W;
    const int g = blockIdx.x / chunks;
    const int h = g * R + (blockIdx.x % chunks) * W + wave % W;
    const int64_t QB = 64 * QW;
    const int64_t Q0 = (int64_t)(gridDim.y - 1 - blockIdx.y) * QB;  // longest rows first
    const int64_t q0 = Q0 + 64 * (wave / W);

    // stationary query fragments (B operand of S^T = K Q^T)
    half8 qf[2][C];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        const int64_t i = q0 + 32 * t + col;
#pragma unroll
        for (int c = 0; c < C; ++c)
            qf[t][c] = (i < n) ? *reinterpret_cast<const half8*>(Q + (i * Hq + h) * D + c * 16 +
                                                                 khalf)
                               : zero8();
    }

    // stages: first the ones on the diagonal ([Q0, qend)), then keys [0, Q0)
    const int64_t qend = (Q0 + QB < n) ? Q0 + QB : n;
    const int nd = (int)((qend - Q0 + KS - 1) / KS);
    const int ns = nd + (int)(Q0 / KS);
    auto key0 = [&](int s) -> int64_t {
        return s < nd ? Q0 + (int64_t)KS * s : (int64_t)KS * (s - nd);
    };

    Stager<D, KS, NT> st;
    const _Float16* Kg = K + (int64_t)g * D;
    const int64_t kstride = (int64_t)Hkv * D;
    auto kload = [&](int s) { st.load(Kg + key0(s) * kstride, n - key0(s), kstride); };
    // prologue: stages 0 and 1 in LDS, stage 2 in flight
    st.init(tid, kstride);
    kload(0);
    st.store(smem);
    if (ns > 1) {
        kload(1);
        st.store(smem + SB);
        if (ns > 2) kload(2);
    }
    __syncthreads();

    float m[2] = {-INFINITY, -INFINITY};
    float s[2] = {0.0f, 0.0f};
    auto next_stage = [&](int si) {
        if (si + 2 < ns) {
            st.store(smem + ((si + 2) % 3) * SB);
            if (si + 3 < ns) kload(si + 3);
        }
        __syncthreads();
    };

    // diagonal stages: causal mask, exact online max
    for (int si = 0; si < nd; ++si) {
        const _Float16* buf = smem + (si % 3) * SB;
        const int64_t k0 = key0(si);
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t kt0 = k0 + 32 * u;
            const bool need0 = kt0 <= q0 + 31;
            const bool need1 = kt0 <= q0 + 63;
            if (!need1) continue;
            floatx16 acc0 = zero16(), acc1 = zero16();
            const _Float16* arow = buf + (32 * u + col) * PITCH + khalf;
#pragma unroll
            for (int c = 0; c < C; ++c) {
                const half8 a = *reinterpret_cast<const half8*>(arow + c * 16);
                if (need0) acc0 = mfma32(a, qf[0][c], acc0);
                acc1 = mfma32(a, qf[1][c], acc1);
            }
            const int lim = (int)(q0 - kt0) + col;  // query - first key of the tile
            if (need0) exact_update(acc0, c2, kt0 + 31 > q0, lim, lane, m[0], s[0]);
            exact_update(acc1, c2, kt0 + 31 > q0 + 32, lim + 32, lane, m[1], s[1]);
        }
        next_stage(si);
    }
    // one reference per query row for the remaining stages
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        float mn = fmaxf(m[t], __shfl_xor(m[t], 32, 64));
        if (mn == -INFINITY) mn = 0.0f;
        s[t] = (m[t] == -INFINITY) ? 0.0f : s[t] * ex2(m[t] - mn);
        m[t] = mn;
    }

    // stages strictly below the diagonal: no mask, fixed reference.  The
    // pipeline runs the softmax of each 32-key unit while the MFMAs of the
    // next unit (in this stage or the next) execute, and each key fragment is
    // read from LDS two MFMA steps before its use (the first two of a unit
    // during the previous unit, across a stage boundary too); `pend` starts
    // as -inf, which contributes exactly zero.
    floatx16 pend[2];
#pragma unroll
    for (int e = 0; e < 16; ++e) {
        pend[0][e] = -INFINITY;
        pend[1][e] = -INFINITY;
    }
    const int fo = col * PITCH + khalf;  // this lane's fragment offset in a unit
    half8 pf[2];                         // the next unit's first two fragments
    if (nd < ns) {
        pf[0] = *reinterpret_cast<const half8*>(smem + (nd % 3) * SB + fo);
        pf[1] = *reinterpret_cast<const half8*>(smem + (nd % 3) * SB + fo + 16);
    }
    for (int si = nd; si < ns; ++si) {
        const _Float16* buf = smem + (si % 3) * SB;
        const _Float16* nbuf = smem + ((si + 1) % 3) * SB;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const _Float16* urow = buf + 32 * u * PITCH + fo;
            const _Float16* nrow = (u + 1 < U) ? urow + 32 * PITCH : nbuf + fo;
            half8 f[C];
            f[0] = pf[0];
            f[1] = pf[1];
            floatx16 cur0 = zero16(), cur1 = zero16();
#pragma unroll
            for (int c = 0; c < C; ++c) {
                if (c + 2 < C)
                    f[c + 2] = *reinterpret_cast<const half8*>(urow + (c + 2) * 16);
                else
                    pf[c + 2 - C] = *reinterpret_cast<const half8*>(nrow + (c + 2 - C) * 16);
                cur0 = mfma32(f[c], qf[0][c], cur0);
                cur1 = mfma32(f[c], qf[1][c], cur1);
            }
            fixed_ref_update(pend, c2, lane, m, s);
            pend[0] = cur0;
            pend[1] = cur1;
        }
        next_stage(si);
    }
    fixed_ref_update(pend, c2, lane, m, s);
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        const float mo = __shfl_xor(m[t], 32, 64);
        const float so = __shfl_xor(s[t], 32, 64);
        const float M = fmaxf(m[t], mo);
        const float tot = ((m[t] == -INFINITY) ? 0.0f : s[t] * ex2(m[t] - M)) +
                          ((mo == -INFINITY) ? 0.0f : so * ex2(mo - M));
        const int64_t i = q0 + 32 * t + col;
        if (lane < 32 && i < n) lse2[(int64_t)h * n + i] = M + log2f(tot);
    }
}

// ---------------------------------------------------------------- pass 2 --
// Pass 2 computes S^T = K Q^T as well: the stationary keys are the A operand
// (the same registers a Q K^T layout would use as B), the streamed queries
// the B operand, so a lane of the C tile owns one query column: one lse value
// per lane and tile, and 16 key rows whose weights add into 16 independent
// per-lane column accumulators (summed across the 32 query lanes once, at the
// end).

// acc[e] += 2^(c2 x_e - L) for the 16 elements of a C tile.
__device__ __forceinline__ void tile_colacc(const floatx16& a, float L, float c2,
                                            float (&acc)[16]) {
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[e] += ex2(fmaf(a[e], c2, -L));
}

// Same on a diagonal tile: only keys at or before the lane's query, i.e. key
// rows crow(e) <= last = query - (first key of the tile).
__device__ __forceinline__ void tile_colacc_masked(const floatx16& a, float L, float c2, int last,
                                                   int lane, float (&acc)[16]) {
#pragma unroll
    for (int e = 0; e < 16; ++e) {
        const float p = ex2(fmaf(a[e], c2, -L));
        acc[e] += (crow(e, lane) <= last) ? p : 0.0f;
    }
}

template <int D, int KW, int QS>
__global__ __launch_bounds__(KW * 64, 2) void colsum_kernel(
    const _Float16* __restrict__ Q, const _Float16* __restrict__ K,
    const float* __restrict__ lse2, float* __restrict__ partial, int64_t n, int64_t ldp, int Hq,
    int Hkv, float c2) {
    constexpr int NT = KW * 64;
    constexpr int C = D / 16;
    constexpr int PITCH = D + 8;
    constexpr int U = QS / 32;  // 32-query units per stage
    constexpr int SB = QS * PITCH;  // halfs per stage buffer
    static_assert(QS <= NT, "one lse value per thread and stage");
    // a ring of three stage buffers [3][QS][PITCH] of query tiles, then float
    // [3][QS] lse values.  Stage s lives in buffer s % 3 and is stored at the
    // end of stage s - 2, before that stage's barrier, so during stage s the
    // buffer of stage s + 1 is already valid (the next stage's first
    // fragments are read ahead) and the buffer written at the end of stage s
    // (that of s + 2, last read in stage s - 1) is no longer read by anyone.
    extern __shared__ _Float16 smem[];
    float* lsm = reinterpret_cast<float*>(smem + 3 * SB);
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int col = lane & 31;
    const int khalf = 8 * (lane >> 5);
    // layer blockIdx.z of an all-layer launch (partial [L][Hq][ldp])
    Q += (int64_t)blockIdx.z * n * Hq * D;
    K += (int64_t)blockIdx.z * n * Hkv * D;
    lse2 += (int64_t)blockIdx.z * Hq * n;
    partial += (int64_t)blockIdx.z * Hq * ldp;
    const int h = blockIdx.x;
    const int g = h / (Hq / Hkv);
    const int64_t K0 = (int64_t)blockIdx.y * (kColKeys * KW);  // blockIdx.y = 0: most work
    const int64_t k0 = K0 + kColKeys * wave;

    // stationary key fragments (A operand of S^T = K Q^T)
    half8 kf[2][C];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        const int64_t j = k0 + 32 * t + col;
#pragma unroll
        for (int c = 0; c < C; ++c)
            kf[t][c] = (j < n) ? *reinterpret_cast<const half8*>(K + (j * Hkv + g) * D + c * 16 +
                                                                 khalf)
                               : zero8();
    }

    const int ns = (int)((n - K0 + QS - 1) / QS);  // query stages from K0 on
    Stager<D, QS, NT> st;
    const _Float16* Qh = Q + (int64_t)h * D;
    const int64_t qstride = (int64_t)Hq * D;
    const float* lrow = lse2 + (int64_t)h * n;
    auto lload = [&](int s) -> float {
        const int64_t i = K0 + (int64_t)QS * s + tid;
        return (tid < QS && i < n) ? lrow[i] : INFINITY;  // no query: weight 2^-inf = 0
    };
    auto qload = [&](int s) {
        const int64_t t0 = K0 + (int64_t)QS * s;
        st.load(Qh + t0 * qstride, n - t0, qstride);
    };
    // prologue: stages 0 and 1 in LDS, stage 2 in flight
    st.init(tid, qstride);
    qload(0);
    float lv = lload(0);
    st.store(smem);
    if (tid < QS) lsm[tid] = lv;
    if (ns > 1) {
        qload(1);
        lv = lload(1);
        st.store(smem + SB);
        if (tid < QS) lsm[QS + tid] = lv;
        if (ns > 2) {
            qload(2);
            lv = lload(2);
        }
    }
    __syncthreads();

    // per key tile t, the column accumulators of the lane's 16 key rows
    float ca[2][16];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int e = 0; e < 16; ++e) ca[t][e] = 0.0f;
    // Software pipeline over the stages after this wavefront's keys: the
    // weights of each 32-query unit are summed while the MFMAs of the next
    // unit execute, and each fragment is read from LDS one MFMA step before
    // its use (the first one of a unit during the previous unit, across a
    // stage boundary too).  `pend` starts as -inf with lse 0, which
    // contributes exactly zero.  At d = 256 the MFMAs of a unit take twice
    // its softmax time and the 32 registers of the pending tiles would leave
    // one wavefront per SIMD, so there each unit is summed right after its
    // own MFMAs and the two wavefronts of a SIMD overlap each other instead.
    constexpr bool kPipe = D != 256;
    floatx16 pend[2];
    // lse of the pending unit's query: read from LDS when the unit's MFMAs
    // are issued, so the softmax one unit later waits on no LDS read
    float pL = 0.0f;
    // fragments are read one MFMA step ahead (two steps fit in the registers,
    // 254 of 256, and measured 1% slower at d = 128, the same at d = 256)
    constexpr int kPf = 1;
    half8 pf[kPf];  // the next unit's first fragment, read ahead
    bool have_pf = false;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
        pend[0][e] = -INFINITY;
        pend[1][e] = -INFINITY;
    }
    for (int si = 0; si < ns; ++si) {
        const _Float16* buf = smem + (si % 3) * SB;
        const _Float16* nbuf = smem + ((si + 1) % 3) * SB;
        const float* lb = lsm + (si % 3) * QS;
        const int64_t s0 = K0 + (int64_t)QS * si;
        if (s0 >= k0 + kColKeys) {
            // every query of the stage is after every key of this wavefront
            if constexpr (kPipe) {
                const int fo = col * PITCH + khalf;  // this lane's fragment offset in a unit
                if (!have_pf) {
#pragma unroll
                    for (int c = 0; c < kPf; ++c)
                        pf[c] = *reinterpret_cast<const half8*>(buf + fo + c * 16);
                }
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const _Float16* urow = buf + 32 * u * PITCH + fo;
                    const _Float16* nrow = (u + 1 < U) ? urow + 32 * PITCH : nbuf + fo;
                    half8 f[C];
#pragma unroll
                    for (int c = 0; c < kPf; ++c) f[c] = pf[c];
                    floatx16 cur0 = zero16(), cur1 = zero16();
#pragma unroll
                    for (int c = 0; c < C; ++c) {
                        if (c + kPf < C)
                            f[c + kPf] = *reinterpret_cast<const half8*>(urow + (c + kPf) * 16);
                        else
                            pf[c + kPf - C] =
                                *reinterpret_cast<const half8*>(nrow + (c + kPf - C) * 16);
                        cur0 = mfma32(kf[0][c], f[c], cur0);
                        cur1 = mfma32(kf[1][c], f[c], cur1);
                    }
                    const float Lnext = lb[32 * u + col];
                    tile_colacc(pend[0], pL, c2, ca[0]);
                    tile_colacc(pend[1], pL, c2, ca[1]);
                    pend[0] = cur0;
                    pend[1] = cur1;
                    pL = Lnext;
                }
                have_pf = true;
            } else {
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    floatx16 cur0 = zero16(), cur1 = zero16();
                    const _Float16* brow = buf + (32 * u + col) * PITCH + khalf;
#pragma unroll
                    for (int c = 0; c < C; ++c) {
                        const half8 b = *reinterpret_cast<const half8*>(brow + c * 16);
                        cur0 = mfma32(kf[0][c], b, cur0);
                        cur1 = mfma32(kf[1][c], b, cur1);
                    }
                    const float L = lb[32 * u + col];
                    tile_colacc(cur0, L, c2, ca[0]);
                    tile_colacc(cur1, L, c2, ca[1]);
                }
            }
        } else if (s0 + QS > k0) {
            // the stage crosses this wavefront's keys: causal mask (these
            // stages precede every full one, so nothing is pending yet)
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int64_t it0 = s0 + 32 * u;
                const bool need0 = k0 <= it0 + 31;
                const bool need1 = k0 + 32 <= it0 + 31;
                if (!need0) continue;
                const float L = lb[32 * u + col];
                floatx16 acc0 = zero16(), acc1 = zero16();
                const _Float16* brow = buf + (32 * u + col) * PITCH + khalf;
#pragma unroll
                for (int c = 0; c < C; ++c) {
                    const half8 b = *reinterpret_cast<const half8*>(brow + c * 16);
                    acc0 = mfma32(kf[0][c], b, acc0);
                    if (need1) acc1 = mfma32(kf[1][c], b, acc1);
                }
                const int last = (int)(it0 - k0) + col;  // query - first key of the tile
                tile_colacc_masked(acc0, L, c2, last, lane, ca[0]);
                if (need1) tile_colacc_masked(acc1, L, c2, last - 32, lane, ca[1]);
            }
        }
        if (si + 2 < ns) {
            st.store(smem + ((si + 2) % 3) * SB);
            if (tid < QS) lsm[((si + 2) % 3) * QS + tid] = lv;
            if (si + 3 < ns) {
                qload(si + 3);
                lv = lload(si + 3);
            }
        }
        __syncthreads();
    }
    if constexpr (kPipe) {
        tile_colacc(pend[0], pL, c2, ca[0]);
        tile_colacc(pend[1], pL, c2, ca[1]);
    }
    // sum each key row over the 32 query lanes of its half by a transpose
    // reduction: at the exchange with lane ^ m (m = 16, 8, 4, 2) a lane keeps
    // one half of its remaining rows (the upper half when lane & m) and adds
    // its partner's copy of them, so 8 + 4 + 2 + 1 exchanges leave row
    // e = (lane >> 1) & 15 summed over 16 lanes, and a last exchange with
    // lane ^ 1 completes it; the even lanes of each half write their row
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        float r8[8], r4[4], r2[2];
        const bool u16 = (col & 16) != 0, u8 = (col & 8) != 0, u4 = (col & 4) != 0,
                   u2 = (col & 2) != 0;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float keep = u16 ? ca[t][i + 8] : ca[t][i];
            const float send = u16 ? ca[t][i] : ca[t][i + 8];
            r8[i] = keep + __shfl_xor(send, 16, 64);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float keep = u8 ? r8[i + 4] : r8[i];
            const float send = u8 ? r8[i] : r8[i + 4];
            r4[i] = keep + __shfl_xor(send, 8, 64);
        }
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const float keep = u4 ? r4[i + 2] : r4[i];
            const float send = u4 ? r4[i] : r4[i + 2];
            r2[i] = keep + __shfl_xor(send, 4, 64);
        }
        float v = (u2 ? r2[1] : r2[0]) + __shfl_xor(u2 ? r2[0] : r2[1], 2, 64);
        v += __shfl_xor(v, 1, 64);
        const int64_t j = k0 + 32 * t + crow((col >> 1) & 15, lane);
        if ((col & 1) == 0 && j < n) partial[(int64_t)h * ldp + j] = v;
    }
}

// score[j] (+)= sum over the P per-head partial rows, added in head order.
// The loads of 8 heads are issued together; the additions stay sequential.
__global__ void reduce_kernel(const float* __restrict__ partial, int64_t ldp, int P,
                              int64_t n, float* __restrict__ score, int acc) {
    const int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (j >= n) return;
    float v = 0.0f;
    int p = 0;
    for (; p + 8 <= P; p += 8) {
        float x[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) x[u] = partial[(int64_t)(p + u) * ldp + j];
#pragma unroll
        for (int u = 0; u < 8; ++u) v += x[u];
    }
    for (; p < P; ++p) v += partial[(int64_t)p * ldp + j];
    score[j] = acc ? score[j] + v : v;
}

// The same over the L layers of an all-layer launch, in two kernels so that
// no thread waits on a chain of L * P loads.  First, for every (token, layer)
// at once, the layer's head sum formed exactly as reduce_kernel forms it,
// written over the layer's partial row 0 (each thread reads and writes only
// its own token's column)...
__global__ void layer_headsum_kernel(float* __restrict__ partial, int64_t ldp, int P,
                                     int64_t n) {
    const int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (j >= n) return;
    float* pl = partial + (int64_t)blockIdx.y * P * ldp;
    float v = 0.0f;
    int p = 0;
    for (; p + 8 <= P; p += 8) {
        float x[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) x[u] = pl[(int64_t)(p + u) * ldp + j];
#pragma unroll
        for (int u = 0; u < 8; ++u) v += x[u];
    }
    for (; p < P; ++p) v += pl[(int64_t)p * ldp + j];
    pl[j] = v;
}

// ...then the layers' sums added to the score in layer order, as a call of
// reduce_kernel per layer (accumulating from the second layer on) adds them,
// so the result is bit-identical to scoring the layers one call at a time.
// ldl = P * ldp is the distance between two layers' row 0.
__global__ void layer_total_kernel(const float* __restrict__ partial, int64_t ldl, int64_t n,
                                   int L, float* __restrict__ score, int acc) {
    const int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (j >= n) return;
    float s = acc ? score[j] : 0.0f;
    int l = 0;
    for (; l + 8 <= L; l += 8) {
        float x[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) x[u] = partial[(int64_t)(l + u) * ldl + j];
#pragma unroll
        for (int u = 0; u < 8; ++u) s = (l + u == 0 && !acc) ? x[u] : s + x[u];
    }
    for (; l < L; ++l) {
        const float x = partial[(int64_t)l * ldl + j];
        s = (l == 0 && !acc) ? x : s + x;
    }
    score[j] = s;
}

// Pass-1 workgroup shape: W heads of a GQA group (the largest of 4, 2, 1
// that divides R = Hq/Hkv) times QW = 4/W blocks of 64 queries, so always
// four wavefronts, one per SIMD, and two workgroups per CU.  (Taking W = R
// for R = 7 gave seven-wavefront workgroups, one per CU, and ran 10% slower
// on the Qwen-shaped heads.)
int rowlse_heads(int R) {
    for (int w = 4; w >= 1; w >>= 1)
        if (R % w == 0) return w;
    return 1;
}

constexpr int rowlse_qblocks(int W) { return 4 / W; }

template <int D>
constexpr int stage_rows() { return D == 256 ? 32 : kStageKeys; }

template <int D, int W>
hipError_t launch_rowlse_t(const Dims& s, const void* q, const void* k, float* lse2,
                           hipStream_t st, int layers) {
    constexpr int QW = rowlse_qblocks(W);
    constexpr int KS = stage_rows<D>();
    const int64_t QB = 64 * QW;
    const dim3 grid((unsigned)(s.Hq / W), (unsigned)((s.n + QB - 1) / QB), (unsigned)layers);
    const float c2 = kLog2e / sqrtf((float)s.d);
    const size_t lds = (size_t)3 * KS * (D + 8) * 2;
    hipLaunchKernelGGL((rowlse_kernel<D, W, QW, KS>), grid, dim3(W * QW * 64), lds, st,
                       (const _Float16*)q, (const _Float16*)k, lse2, s.n, s.Hq, s.Hkv, c2);
    return hipGetLastError();
}

template <int D>
hipError_t launch_rowlse_d(const Dims& s, const void* q, const void* k, float* lse2,
                           hipStream_t st, int layers) {
    switch (rowlse_heads(s.Hq / s.Hkv)) {
        case 1: return launch_rowlse_t<D, 1>(s, q, k, lse2, st, layers);
        case 2: return launch_rowlse_t<D, 2>(s, q, k, lse2, st, layers);
        case 4: return launch_rowlse_t<D, 4>(s, q, k, lse2, st, layers);
        default: return hipErrorInvalidValue;
    }
}

template <int D>
hipError_t launch_colsum_d(const Dims& s, const void* q, const void* k, const float* lse2,
                           float* partial, hipStream_t st, int layers) {
    constexpr int QS = stage_rows<D>();
    const int64_t KB = (int64_t)kColKeys * kColWaves;
    const dim3 grid((unsigned)s.Hq, (unsigned)((s.n + KB - 1) / KB), (unsigned)layers);
    const float c2 = kLog2e / sqrtf((float)s.d);
    const size_t lds = (size_t)3 * QS * (D + 8) * 2 + (size_t)3 * QS * 4;
    hipLaunchKernelGGL((colsum_kernel<D, kColWaves, QS>), grid, dim3(kColWaves * 64), lds, st,
                       (const _Float16*)q, (const _Float16*)k, lse2, partial, s.n,
                       padded_tokens(s.n), s.Hq, s.Hkv, c2);
    return hipGetLastError();
}

}  // namespace

int64_t padded_tokens(int64_t n) { return (n + kColKeys - 1) / kColKeys * kColKeys; }

hipError_t launch_rowlse(const Dims& s, const void* q, const void* k, float* lse2,
                         hipStream_t st, int layers) {
    switch (s.d) {
        case 64: return launch_rowlse_d<64>(s, q, k, lse2, st, layers);
        case 128: return launch_rowlse_d<128>(s, q, k, lse2, st, layers);
        case 256: return launch_rowlse_d<256>(s, q, k, lse2, st, layers);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_colsum(const Dims& s, const void* q, const void* k, const float* lse2,
                         float* partial, hipStream_t st, int layers) {
    switch (s.d) {
        case 64: return launch_colsum_d<64>(s, q, k, lse2, partial, st, layers);
        case 128: return launch_colsum_d<128>(s, q, k, lse2, partial, st, layers);
        case 256: return launch_colsum_d<256>(s, q, k, lse2, partial, st, layers);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_reduce(const Dims& s, const float* partial, float* score, int acc,
                         hipStream_t st) {
    const unsigned blocks = (unsigned)((s.n + 255) / 256);
    hipLaunchKernelGGL(reduce_kernel, dim3(blocks), dim3(256), 0, st, partial,
                       padded_tokens(s.n), s.Hq, s.n, score, acc);
    return hipGetLastError();
}

hipError_t launch_reduce_layers(const Dims& s, float* partial, float* score, int acc,
                                hipStream_t st, int layers) {
    const unsigned blocks = (unsigned)((s.n + 255) / 256);
    const int64_t ldp = padded_tokens(s.n);
    hipLaunchKernelGGL(layer_headsum_kernel, dim3(blocks, (unsigned)layers), dim3(256), 0, st,
                       partial, ldp, s.Hq, s.n);
    hipLaunchKernelGGL(layer_total_kernel, dim3(blocks), dim3(256), 0, st,
                       (const float*)partial, (int64_t)s.Hq * ldp, s.n, layers, score, acc);
    return hipGetLastError();
}

int colsum_partial_rows(const Dims& s) { return s.Hq; }

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

hipError_t score_scratch(void** ptr, size_t* bytes) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    *bytes = sizeof(scratch);
    return hipSuccess;
}

}  // namespace sk
