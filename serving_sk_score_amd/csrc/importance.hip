// Score variants of the SpectrumKV paper's Algorithm 1 "score tokens": the
// recency factor of the §4.3 importance formula and the KV-norm fallback.
//
// Recency: an elementwise pass, one thread per token, in double precision so
// that lambda * Delta_j stays exact for every n < 2^30 and the only roundings
// are exp's and the final one to fp32.
//
// KV-norm: score_j = sum over layers l and KV heads g of ||k[l][j][g]||_2.
// It streams every key once (n * L * H * d fp16 values) and is bound by HBM.
// Mapping: one wavefront per token.  A token's slice of one layer is H rows of
// d elements, contiguous in memory; the wave reads it as 16-byte pieces, a
// row spread over G = d/8 neighbouring lanes (one "row group"), so every load
// instruction is a fully coalesced 1 KiB.  A wave step covers 64 pieces; the
// wave walks the L * ceil(H*G / 64) steps of its token NB at a time, all NB
// loads in flight before any arithmetic.
//
// Row sums of squares are needed once per row, so the NB per-lane partial
// sums of a batch (NB different rows of one row group) are reduced together
// with a transpose reduction: at each of log2(NB) exchanges a lane keeps half
// of its values, sends the other half to its partner and adds what it
// receives, so NB values need NB - 1 exchanges instead of NB * log2(G).
// Afterwards every lane holds one complete row sum (each row held by G/NB
// lanes), takes its square root and adds it to a running total; the wave's
// total is scaled by NB/G (an exact power of two) at the end.
#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>

#include "sk_kernels.h"

namespace sk {
namespace {

constexpr int kWaves = 4;  // wavefronts (tokens) per workgroup

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ u32x4 ld_nt(const uint16_t* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

// value of lane (lane ^ S) within each group of 32 lanes (S < 32)
template <int S>
__device__ __forceinline__ float swz_xor(float x) {
    static_assert(S > 0 && S < 32, "swizzle xor mask");
    return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(x), 0x1F | (S << 10)));
}

__device__ __forceinline__ float sq_lo(uint32_t w, float acc) {
    const float x = __half2float(__ushort_as_half((unsigned short)(w & 0xFFFFu)));
    return fmaf(x, x, acc);  // x*x is exact in fp32 for fp16 x
}
__device__ __forceinline__ float sq_hi(uint32_t w, float acc) {
    const float x = __half2float(__ushort_as_half((unsigned short)(w >> 16)));
    return fmaf(x, x, acc);
}

__device__ __forceinline__ float sumsq8(u32x4 r) {
    float s = 0.0f;
    s = sq_lo(r.x, s);
    s = sq_hi(r.x, s);
    s = sq_lo(r.y, s);
    s = sq_hi(r.y, s);
    s = sq_lo(r.z, s);
    s = sq_hi(r.z, s);
    s = sq_lo(r.w, s);
    s = sq_hi(r.w, s);
    return s;
}

// One exchange of the transpose reduction over K values with lane mask S:
// the lane whose S bit is clear keeps v[0..K/2), the other keeps v[K/2..K);
// each adds its partner's copy of the half it keeps.
template <int S, int K>
__device__ __forceinline__ void transpose_step(float (&v)[8], int lane) {
    const bool hi = (lane & S) != 0;
#pragma unroll
    for (int t = 0; t < K / 2; ++t) {
        const float a = v[t], b = v[t + K / 2];
        const float send = hi ? a : b;
        const float keep = hi ? b : a;
        v[t] = keep + swz_xor<S>(send);
    }
}

template <int D>
__device__ __forceinline__ float row_sum_of_batch(float (&v)[8], int lane) {
    constexpr int G = D / 8;  // lanes per row: 8, 16 or 32
    transpose_step<G / 2, 8>(v, lane);
    transpose_step<G / 4, 4>(v, lane);
    transpose_step<G / 8, 2>(v, lane);
    float s = v[0];
    if constexpr (G >= 16) s += swz_xor<G / 16>(s);
    if constexpr (G >= 32) s += swz_xor<G / 32>(s);
    return s;
}

__device__ __forceinline__ int64_t wave_token() {
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    return (int64_t)blockIdx.x * kWaves + w;
}

template <int D>
__global__ __launch_bounds__(kWaves * 64) void kvnorm_kernel(
    const uint16_t* __restrict__ K, float* __restrict__ score, int64_t n, int H, int L,
    int accumulate) {
    constexpr int NB = 8;      // wave steps per batch
    constexpr int G = D / 8;   // lanes per row
    const int lane = threadIdx.x & 63;
    const int64_t j = wave_token();
    if (j >= n) return;
    const int P = H * G;               // 16-byte pieces of one layer's slice
    const int PPL = (P + 63) / 64;     // wave steps per layer
    const int M = L * PPL;             // wave steps of the token
    const int64_t lstride = n * (int64_t)H * D;
    const uint16_t* base = K + j * (int64_t)H * D;

    float total = 0.0f;
    int layer = 0, step = 0;  // layer and step within the layer of step m0 + t
    for (int m0 = 0; m0 < M; m0 += NB) {
        u32x4 raw[NB];
        bool ok[NB];
#pragma unroll
        for (int t = 0; t < NB; ++t) {
            const int p = step * 64 + lane;
            ok[t] = (m0 + t < M) && (p < P);
            // out-of-range steps and lanes load an in-range piece and discard it
            const int pc = p < P ? p : P - 1;
            const int lc = layer < L ? layer : L - 1;
            raw[t] = ld_nt(base + lc * lstride + (int64_t)pc * 8);
            if (++step == PPL) {
                step = 0;
                ++layer;
            }
        }
        float v[NB];
#pragma unroll
        for (int t = 0; t < NB; ++t) {
            const float s = sumsq8(raw[t]);
            v[t] = ok[t] ? s : 0.0f;
        }
        total += sqrtf(row_sum_of_batch<D>(v, lane));
    }
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) total += __shfl_xor(total, m, 64);
    total *= (float)NB / (float)G;
    if (lane == 0) score[j] = accumulate ? score[j] + total : total;
}

__global__ __launch_bounds__(256) void recency_kernel(const float* in, float* out, int64_t n,
                                                      double lambda) {
    const int64_t j = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (j >= n) return;
    const double w = exp(-lambda * (double)(n - 1 - j));
    out[j] = (float)((double)in[j] * w);
}

}  // namespace

hipError_t launch_kvnorm(const Dims& s, const void* k, float* score, int accumulate,
                         hipStream_t st) {
    const dim3 grid((unsigned)((s.n + kWaves - 1) / kWaves));
    const uint16_t* K = static_cast<const uint16_t*>(k);
    switch (s.d) {
        case 64:
            kvnorm_kernel<64><<<grid, kWaves * 64, 0, st>>>(K, score, s.n, s.Hkv, s.L, accumulate);
            break;
        case 128:
            kvnorm_kernel<128><<<grid, kWaves * 64, 0, st>>>(K, score, s.n, s.Hkv, s.L, accumulate);
            break;
        case 256:
            kvnorm_kernel<256><<<grid, kWaves * 64, 0, st>>>(K, score, s.n, s.Hkv, s.L, accumulate);
            break;
        default:
            return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_recency(int64_t n, double lambda, const float* in, float* out,
                          hipStream_t st) {
    const dim3 grid((unsigned)((n + 255) / 256));
    recency_kernel<<<grid, 256, 0, st>>>(in, out, n, lambda);
    return hipGetLastError();
}

}  // namespace sk
