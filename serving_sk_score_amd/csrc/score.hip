// Token importance score: causal attention column sums with MFMA.
//
// SpectrumKV paper, §4.3 (I_j = A_j exp(-lambda Delta_j), here lambda = 0) and
// Algorithm 1 "score tokens"; the score is the attention a token receives,
// summed over query heads (and, across calls, layers):
//     A_j = sum_h sum_{i >= j} softmax_i(q_i . k_j / sqrt(d))_j.
//
// The softmax of row i needs the whole row before any column can be summed,
// and storing P is O(n^2), so the path is two passes over Q K^T:
//   pass 1 (rowlse): lse[h][i] = ln sum_{j<=i} exp(s_ij), online max/sum;
//   pass 2 (colsum): recompute s_ij and sum exp(s_ij - lse_i) down each
//                    column j, per KV head group; a fixed-order reduction over
//                    groups then yields the layer's A_j.
// Both passes are dense fp16 contractions on v_mfma_f32_32x32x16_f16 with
// fp32 accumulation; the softmax arithmetic is fp32 in base 2
// (exp2(s * log2(e)/sqrt(d) - m)).
//
// MFMA 32x32x16 operand layout (per 64-lane wavefront):
//   A (32 x 16): lane l holds row l%32, k = 8*(l/32) .. +7
//   B (16 x 32): lane l holds column l%32, k = 8*(l/32) .. +7
//   C (32 x 32): lane l holds column l%32, rows 8*(e/4) + 4*(l/32) + e%4, e = 0..15
// A and B are both "k-contiguous", which is exactly the row-major [token][d]
// layout of Q and K, so fragments are single 16-byte reads.
//
// pass 1 computes S^T = K Q^T (rows = keys, columns = queries): each lane owns
// one query and 16 of the 32 keys of a tile, so the row max / row sum are
// in-lane plus one exchange with lane l^32.  A workgroup is the W query heads
// of one GQA group (one wavefront each) over the same 64 queries, so each K
// tile is staged once in LDS and read by all W heads.
//
// pass 2 computes S = Q K^T (rows = queries, columns = keys): each lane owns
// one key column of each 32-key sub-tile, so the column sum is an in-lane
// accumulation across all query tiles.  A workgroup keeps 64 keys of its
// group stationary in registers (one wavefront per query head) and streams
// the W heads' query tiles through LDS.
//
// Work is causal (tile pairs above the diagonal are skipped) and workgroups
// are launched longest-first; the KV group index runs fastest across the
// grid so that consecutive workgroups (round-robin over the 8 XCDs) of one
// group land on the same XCD and share its L2.
#include <hip/hip_runtime.h>

#include "sk_kernels.h"

namespace sk {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

constexpr int kMaxWaves = 8;
constexpr int kQB = 64;   // queries per pass-1 workgroup (2 sub-tiles)
constexpr int kKB = 64;   // keys per pass-2 workgroup (2 sub-tiles)
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ floatx16 mfma32(half8 a, half8 b, floatx16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ half8 zero8() {
    half8 z;
#pragma unroll
    for (int e = 0; e < 8; ++e) z[e] = (_Float16)0.0f;
    return z;
}

// Row within a 32x32 C tile held by element e of lane l.
__device__ __forceinline__ int crow(int e, int lane) {
    return 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
}

// Cooperative staging of 32 tokens x NSEG*D halfs (contiguous per token in
// global memory, token stride `gstride` halfs) into LDS rows of D + 8 halfs
// by NT threads.  LDS row index = seg * 32 + token (seg-major), so that the
// MFMA fragment reads of 32 consecutive LDS rows at a fixed column are
// bank-conflict free (row pitch = 4 banks mod 64).
template <int D, int NSEG, int NT>
struct Stager {
    static constexpr int kPieces = D / 8;                 // 16-byte pieces per segment
    static constexpr int kTotal = 32 * NSEG * kPieces;
    static constexpr int kRegs = (kTotal + NT - 1) / NT;
    uint4 regs[kRegs];
    __device__ void load(int tid, const _Float16* __restrict__ g, int64_t t0, int64_t n,
                         int64_t gstride) {
#pragma unroll
        for (int r = 0; r < kRegs; ++r) {
            const int idx = tid + r * NT;
            uint4 v = make_uint4(0, 0, 0, 0);
            if (kTotal % NT == 0 || idx < kTotal) {
                const int tok = idx / (NSEG * kPieces);
                const int rem = idx % (NSEG * kPieces);
                if (t0 + tok < n)
                    v = *reinterpret_cast<const uint4*>(g + (t0 + tok) * gstride + rem * 8);
            }
            regs[r] = v;
        }
    }
    __device__ void store(int tid, _Float16* lds) const {
#pragma unroll
        for (int r = 0; r < kRegs; ++r) {
            const int idx = tid + r * NT;
            if (kTotal % NT == 0 || idx < kTotal) {
                const int tok = idx / (NSEG * kPieces);
                const int rem = idx % (NSEG * kPieces);
                const int seg = rem / kPieces, piece = rem % kPieces;
                *reinterpret_cast<uint4*>(lds + (seg * 32 + tok) * (D + 8) + piece * 8) =
                    regs[r];
            }
        }
    }
};

// ---------------------------------------------------------------- pass 1 --
template <int D, int W>
__global__ __launch_bounds__(W * 64) void rowlse_kernel(
    const _Float16* __restrict__ Q, const _Float16* __restrict__ K, float* __restrict__ lse,
    int64_t n, int Hq, int Hkv, float c2) {
    extern __shared__ _Float16 smem[];  // [32][D + 8]
    constexpr int C = D / 16;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int R = Hq / Hkv;
    const int chunks = R / W;
    const int g = blockIdx.x / chunks;
    const int h = g * R + (blockIdx.x % chunks) * W + wave;
    const int64_t nqb = gridDim.y;
    const int64_t qb = nqb - 1 - blockIdx.y;  // longest rows first
    const int64_t q0 = qb * kQB;

    // stationary query fragments (B operand of S^T = K Q^T)
    half8 qf[2][C];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        const int64_t i = q0 + 32 * t + (lane & 31);
#pragma unroll
        for (int c = 0; c < C; ++c) {
            qf[t][c] = (i < n) ? *reinterpret_cast<const half8*>(
                                     Q + (i * Hq + h) * D + c * 16 + 8 * (lane >> 5))
                               : zero8();
        }
    }

    Stager<D, 1, W * 64> st;
    const int tid = threadIdx.x;
    const _Float16* Kg = K + (int64_t)g * D;
    const int64_t kstride = (int64_t)Hkv * D;

    const int64_t last_q = (q0 + kQB < n ? q0 + kQB : n) - 1;
    const int64_t nkt = last_q / 32 + 1;  // key tiles 0 .. nkt-1

    float m[2] = {-INFINITY, -INFINITY};
    float sum[2] = {0.0f, 0.0f};

    st.load(tid, Kg, 0, n, kstride);
    for (int64_t kt = 0; kt < nkt; ++kt) {
        __syncthreads();
        st.store(tid, smem);
        __syncthreads();
        if (kt + 1 < nkt) st.load(tid, Kg, (kt + 1) * 32, n, kstride);

        floatx16 acc[2];
        const bool need[2] = {kt <= 2 * qb, kt <= 2 * qb + 1};
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[t][e] = 0.0f;
        const _Float16* arow = smem + (lane & 31) * (D + 8) + 8 * (lane >> 5);
#pragma unroll
        for (int c = 0; c < C; ++c) {
            const half8 a = *reinterpret_cast<const half8*>(arow + c * 16);
            if (need[0]) acc[0] = mfma32(a, qf[0][c], acc[0]);
            if (need[1]) acc[1] = mfma32(a, qf[1][c], acc[1]);
        }
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            if (!need[t]) continue;
            const bool diag = (kt == 2 * qb + t);
            const int qcol = lane & 31;  // query offset within the tile
            float x[16];
            float mx = -INFINITY;
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                x[e] = acc[t][e];
                if (diag && crow(e, lane) > qcol) x[e] = -INFINITY;
                mx = fmaxf(mx, x[e]);
            }
            mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
            const float mnew = fmaxf(m[t], mx * c2);
            float s = sum[t] * fast_exp2(m[t] - mnew);
#pragma unroll
            for (int e = 0; e < 16; ++e) s += fast_exp2(fmaf(x[e], c2, -mnew));
            sum[t] = s;
            m[t] = mnew;
        }
    }
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        const float tot = sum[t] + __shfl_xor(sum[t], 32, 64);
        const int64_t i = q0 + 32 * t + (lane & 31);
        if (lane < 32 && i < n) lse[(int64_t)h * n + i] = (m[t] + __log2f(tot)) * kLn2;
    }
}

// ---------------------------------------------------------------- pass 2 --
template <int D, int W>
__global__ __launch_bounds__(W * 64) void colsum_kernel(
    const _Float16* __restrict__ Q, const _Float16* __restrict__ K,
    const float* __restrict__ lse, float* __restrict__ partial, int64_t n, int64_t ldp,
    int Hq, int Hkv, float c2) {
    extern __shared__ _Float16 smem[];  // [W][32][D + 8], then float [W][64]
    constexpr int C = D / 16;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int R = Hq / Hkv;
    const int chunks = R / W;
    const int g = blockIdx.x / chunks;
    const int hbase = g * R + (blockIdx.x % chunks) * W;
    const int h = hbase + wave;
    const int64_t k0 = (int64_t)blockIdx.y * kKB;  // blockIdx.y = 0 has the most work

    // stationary key fragments (B operand of S = Q K^T)
    half8 kf[2][C];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        const int64_t j = k0 + 32 * t + (lane & 31);
#pragma unroll
        for (int c = 0; c < C; ++c) {
            kf[t][c] = (j < n) ? *reinterpret_cast<const half8*>(
                                     K + (j * Hkv + g) * D + c * 16 + 8 * (lane >> 5))
                               : zero8();
        }
    }

    Stager<D, W, W * 64> st;
    const int tid = threadIdx.x;
    const _Float16* Qg = Q + (int64_t)hbase * D;
    const int64_t qstride = (int64_t)Hq * D;
    const float* lrow = lse + (int64_t)h * n;

    const int64_t it0 = k0 / 32;             // first query tile (diagonal of sub-tile 0)
    const int64_t nit = (n + 31) / 32;       // query tiles it0 .. nit-1
    float col[2] = {0.0f, 0.0f};

    st.load(tid, Qg, it0 * 32, n, qstride);
    const bool aligned4 = (((int64_t)h * n) & 3) == 0;
    for (int64_t it = it0; it < nit; ++it) {
        __syncthreads();
        st.store(tid, smem);
        __syncthreads();
        if (it + 1 < nit) st.load(tid, Qg, (it + 1) * 32, n, qstride);

        const int64_t i0 = it * 32;
        // base-2 log-sum-exp of this lane's 16 rows
        float L2[16];
        const bool full = (i0 + 32 <= n) && aligned4;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const int r = 8 * b + 4 * (lane >> 5);
            if (full) {
                const float4 v = *reinterpret_cast<const float4*>(lrow + i0 + r);
                L2[4 * b + 0] = v.x * kLog2e;
                L2[4 * b + 1] = v.y * kLog2e;
                L2[4 * b + 2] = v.z * kLog2e;
                L2[4 * b + 3] = v.w * kLog2e;
            } else {
#pragma unroll
                for (int u = 0; u < 4; ++u)
                    L2[4 * b + u] = (i0 + r + u < n) ? lrow[i0 + r + u] * kLog2e : INFINITY;
            }
        }
        const bool need1 = (it > it0);  // sub-tile 1 keys start 32 after i0 of the first tile
        floatx16 acc[2];
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[t][e] = 0.0f;
        const _Float16* arow = smem + (wave * 32 + (lane & 31)) * (D + 8) + 8 * (lane >> 5);
#pragma unroll
        for (int c = 0; c < C; ++c) {
            const half8 a = *reinterpret_cast<const half8*>(arow + c * 16);
            acc[0] = mfma32(a, kf[0][c], acc[0]);
            if (need1) acc[1] = mfma32(a, kf[1][c], acc[1]);
        }
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            if (t == 1 && !need1) continue;
            const int64_t j0 = k0 + 32 * t;
            const bool diag = (i0 == j0);
            const int jc = lane & 31;
            float s = 0.0f;
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                float p = fast_exp2(fmaf(acc[t][e], c2, -L2[e]));
                if (diag && crow(e, lane) < jc) p = 0.0f;
                s += p;
            }
            col[t] += s;
        }
    }
    // combine the two half-waves, then the W heads in a fixed order
    float* red = reinterpret_cast<float*>(smem + (size_t)W * 32 * (D + 8));
    __syncthreads();
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        const float v = col[t] + __shfl_xor(col[t], 32, 64);
        if (lane < 32) red[wave * 64 + 32 * t + lane] = v;
    }
    __syncthreads();
    if (wave == 0) {
        float v = 0.0f;
        for (int w = 0; w < W; ++w) v += red[w * 64 + lane];
        const int64_t j = k0 + lane;
        if (j < n) partial[(int64_t)(blockIdx.x) * ldp + j] = v;
    }
}

__global__ void reduce_kernel(const float* __restrict__ partial, int64_t ldp, int P,
                              int64_t n, float* __restrict__ score, int acc) {
    const int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (j >= n) return;
    float v = 0.0f;
    for (int p = 0; p < P; ++p) v += partial[(int64_t)p * ldp + j];
    score[j] = acc ? score[j] + v : v;
}

// Heads per workgroup: the largest divisor of R = Hq/Hkv that keeps the
// workgroup within 8 wavefronts (4 for d = 256) and the pass's LDS staging
// within 64 KiB.
int heads_per_wg(int R, int D, bool pass2) {
    for (int w = kMaxWaves; w >= 1; --w) {
        if (R % w) continue;
        if (D == 256 && w > 4) continue;  // register budget of the d=256 fragments
        const size_t lds = pass2 ? (size_t)w * 32 * (D + 8) * 2 + (size_t)w * 64 * 4
                                 : (size_t)32 * (D + 8) * 2;
        if (lds <= 64 * 1024) return w;
    }
    return 1;
}

template <typename F>
hipError_t dispatch_dw(int d, int w, F&& f) {
#define SK_W_CASES(DV)                                                   \
    switch (w) {                                                         \
        case 1: return f(std::integral_constant<int, DV>{}, std::integral_constant<int, 1>{}); \
        case 2: return f(std::integral_constant<int, DV>{}, std::integral_constant<int, 2>{}); \
        case 3: return f(std::integral_constant<int, DV>{}, std::integral_constant<int, 3>{}); \
        case 4: return f(std::integral_constant<int, DV>{}, std::integral_constant<int, 4>{}); \
        case 5: return f(std::integral_constant<int, DV>{}, std::integral_constant<int, 5>{}); \
        case 6: return f(std::integral_constant<int, DV>{}, std::integral_constant<int, 6>{}); \
        case 7: return f(std::integral_constant<int, DV>{}, std::integral_constant<int, 7>{}); \
        case 8: return f(std::integral_constant<int, DV>{}, std::integral_constant<int, 8>{}); \
        default: return hipErrorInvalidValue;                            \
    }
    switch (d) {
        case 64: SK_W_CASES(64)
        case 128: SK_W_CASES(128)
        case 256: SK_W_CASES(256)
        default: return hipErrorInvalidValue;
    }
#undef SK_W_CASES
}

}  // namespace

int64_t padded_tokens(int64_t n) { return (n + kKB - 1) / kKB * kKB; }

hipError_t launch_rowlse(const Dims& s, const void* q, const void* k, float* lse,
                         hipStream_t st) {
    const int R = s.Hq / s.Hkv;
    const int W = heads_per_wg(R, s.d, false);
    const dim3 grid((unsigned)(s.Hq / W), (unsigned)((s.n + kQB - 1) / kQB));
    const float c2 = kLog2e / sqrtf((float)s.d);
    return dispatch_dw(s.d, W, [&](auto Dc, auto Wc) {
        constexpr int D = decltype(Dc)::value;
        constexpr int WW = decltype(Wc)::value;
        const size_t lds = (size_t)32 * (D + 8) * 2;
        hipLaunchKernelGGL((rowlse_kernel<D, WW>), grid, dim3(WW * 64), lds, st,
                           (const _Float16*)q, (const _Float16*)k, lse, s.n, s.Hq, s.Hkv, c2);
        return hipGetLastError();
    });
}

hipError_t launch_colsum(const Dims& s, const void* q, const void* k, const float* lse,
                         float* partial, hipStream_t st) {
    const int R = s.Hq / s.Hkv;
    const int W = heads_per_wg(R, s.d, true);
    const dim3 grid((unsigned)(s.Hq / W), (unsigned)((s.n + kKB - 1) / kKB));
    const float c2 = kLog2e / sqrtf((float)s.d);
    const int64_t ldp = padded_tokens(s.n);
    return dispatch_dw(s.d, W, [&](auto Dc, auto Wc) {
        constexpr int D = decltype(Dc)::value;
        constexpr int WW = decltype(Wc)::value;
        const size_t lds = (size_t)WW * 32 * (D + 8) * 2 + (size_t)WW * 64 * 4;
        hipLaunchKernelGGL((colsum_kernel<D, WW>), grid, dim3(WW * 64), lds, st,
                           (const _Float16*)q, (const _Float16*)k, lse, partial, s.n, ldp,
                           s.Hq, s.Hkv, c2);
        return hipGetLastError();
    });
}

hipError_t launch_reduce(const Dims& s, const float* partial, float* score, int acc,
                         hipStream_t st) {
    const int R = s.Hq / s.Hkv;
    const int W = heads_per_wg(R, s.d, true);
    const int P = s.Hq / W;
    const int64_t ldp = padded_tokens(s.n);
    const unsigned blocks = (unsigned)((s.n + 255) / 256);
    hipLaunchKernelGGL(reduce_kernel, dim3(blocks), dim3(256), 0, st, partial, ldp, P, s.n,
                       score, acc);
    return hipGetLastError();
}

int colsum_partial_rows(const Dims& s) {
    return s.Hq / heads_per_wg(s.Hq / s.Hkv, s.d, true);
}

}  // namespace sk
