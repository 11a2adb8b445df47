// Tier assignment: sink pinning + importance-sorted fp16/int8/int4 split.
//
// SpectrumKV paper, §7.4.1 and Algorithm 1: the first S tokens are pinned to
// fp16 before ranking; the others are sorted by importance and filled into
// fp16, int8 and (optionally) int4 with the counts of the §4.4 budget mapping.
// §2.3 Proposition 1: any such sorted assignment minimises the
// importance-weighted error for fixed counts.  Ties go to the lower token
// index.
//
// Method.  A token's rank only matters through three thresholds: the k1-th,
// k2-th and k3-th largest key among the non-sink tokens, k1 = n16 - S',
// k2 = k1 + n8, k3 = k2 + n4 (k3 < R only when the plan drops tokens).
// Keys are unique integers key = (score bits << b) | (2^b - 1 - j), where
// b = bits needed to hold n, so a larger key means a higher score or, on a
// tie, a lower index; for non-negative floats the IEEE bit pattern is
// monotone.  The thresholds strictly inside (0, R) are found with one
// MSB-first radix select (8-bit digits, LDS histograms, one workgroup) - each
// pass narrows the prefixes of all of them at once, and a threshold whose
// prefix already matches a single key is settled.  A token is fp16 iff
// key >= K_k1, else int8 iff key >= K_k2, else int4 iff key >= K_k3, else
// dropped.  Slots (positions among the same tier in token order) come from
// per-wavefront tier counts (ballots), one workgroup scan of them per round
// and ballot prefixes within each 64-token step; order[] is the inverse
// permutation, dropped tokens last.
//
// Histogram contention: the top digits of nearby scores coincide, so every
// thread first merges runs of equal digits in registers and issues one LDS
// atomic per run.
#include <hip/hip_runtime.h>

#include "sk_kernels.h"

namespace sk {
namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;

__device__ __forceinline__ uint64_t make_key(float s, int64_t j, int bits) {
    uint32_t u = __float_as_uint(s);
    if (u == 0x80000000u) u = 0u;  // -0.0 ranks as +0.0
    return ((uint64_t)u << bits) | (uint64_t)(((int64_t)1 << bits) - 1 - j);
}

// Within one wavefront: given 256 bins, find the digit D (scanning from the
// top) where the cumulative count first reaches k.  Returns D and the count
// of keys strictly above D.
__device__ void find_digit(const uint32_t* hist, uint64_t k, int lane, int* out_digit,
                           uint64_t* out_above) {
    // lane holds digits 255-4*lane .. 252-4*lane (descending)
    uint32_t c[4];
    uint32_t tot = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        c[e] = hist[255 - 4 * lane - e];
        tot += c[e];
    }
    // inclusive prefix over lanes (lane 0 = highest digits)
    uint32_t incl = tot;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        uint32_t v = __shfl_up(incl, o, 64);
        if (lane >= o) incl += v;
    }
    const uint32_t excl = incl - tot;
    const bool here = (excl < k) && (incl >= k);
    const unsigned long long who = __ballot(here);
    const int src = __ffsll((long long)who) - 1;
    if (lane == src) {
        uint32_t run = excl;
        int digit = 0;
        uint32_t above = excl;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            if (run + c[e] >= k) {
                digit = 255 - 4 * lane - e;
                above = run;
                break;
            }
            run += c[e];
        }
        *out_digit = digit;
        *out_above = above;
    }
}

// Steps of 64 tokens per wavefront and round in the slot pass (2 bits of
// tier per step are kept in one 32-bit register, so at most 16).
constexpr int kChunk = 16;
constexpr int kBatch = 8;  // score loads in flight per thread

__global__ __launch_bounds__(kThreads) void select_kernel(
    const float* __restrict__ score, int64_t n, int64_t sinks, int64_t k1, int64_t k2,
    int64_t k3, int64_t n16, int64_t n8, int64_t n4, uint32_t* __restrict__ map,
    uint32_t* __restrict__ order) {
    constexpr int NS = 3;  // thresholds
    __shared__ uint32_t hist[NS][256];
    __shared__ uint64_t prefix[NS];
    __shared__ uint64_t krem[NS];
    __shared__ int sel_digit[NS];
    __shared__ uint64_t sel_above[NS];
    __shared__ int live[NS];
    __shared__ uint32_t wtot[kWaves][4];
    __shared__ uint32_t running[4];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int64_t R = n - sinks;

    int bits = 1;
    while (((int64_t)1 << bits) < n) ++bits;
    const int total_bits = 32 + bits;
    const int passes = (total_bits + 7) / 8;

    // cond_s(key) = rank < k_s: false for k_s <= 0, true for k_s >= R, else
    // a radix-selected threshold
    const int64_t ks[NS] = {k1, k2, k3};
    if (tid == 0) {
        for (int s = 0; s < NS; ++s) {
            live[s] = ks[s] >= 1 && ks[s] < R;
            prefix[s] = 0;
            krem[s] = (uint64_t)(live[s] ? ks[s] : 1);
        }
    }
    __syncthreads();
    uint64_t pmask = 0;  // bits of the key fixed so far (uniform)

    // A threshold stops being narrowed once its prefix matches a single key:
    // that key is then the only one with the prefix, so comparing with the
    // prefix (low bits zero) ranks every key exactly as comparing with the
    // key itself.  With distinct scores this ends the search within the
    // score bits, before the index bits.
    for (int p = 0; p < passes; ++p) {
        bool active[NS];
#pragma unroll
        for (int s = 0; s < NS; ++s) active[s] = live[s] != 0;
        if (!(active[0] || active[1] || active[2])) break;
        const int shift = 8 * (passes - 1 - p);
        for (int i = tid; i < NS * 256; i += kThreads) (&hist[0][0])[i] = 0;
        __syncthreads();
        uint64_t pre[NS];
        int run_d[NS];
        uint32_t run_c[NS];
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            pre[s] = prefix[s];
            run_d[s] = -1;
            run_c[s] = 0;
        }
        // this thread's tokens sinks + tid, + kThreads, ... in that order,
        // kBatch loads issued before any is used
        for (int64_t jb = sinks + tid; jb < n; jb += (int64_t)kThreads * kBatch) {
            float sv[kBatch];
#pragma unroll
            for (int u = 0; u < kBatch; ++u) {
                const int64_t j = jb + (int64_t)u * kThreads;
                sv[u] = j < n ? score[j] : 0.0f;
            }
#pragma unroll
            for (int u = 0; u < kBatch; ++u) {
                const int64_t j = jb + (int64_t)u * kThreads;
                if (j < n) {
                    const uint64_t key = make_key(sv[u], j, bits);
                    const int dg = (int)((key >> shift) & 0xFFu);
#pragma unroll
                    for (int s = 0; s < NS; ++s) {
                        if (active[s] && (key & pmask) == pre[s]) {
                            if (dg != run_d[s]) {
                                if (run_c[s]) atomicAdd(&hist[s][run_d[s]], run_c[s]);
                                run_d[s] = dg;
                                run_c[s] = 0;
                            }
                            ++run_c[s];
                        }
                    }
                }
            }
        }
#pragma unroll
        for (int s = 0; s < NS; ++s)
            if (run_c[s]) atomicAdd(&hist[s][run_d[s]], run_c[s]);
        __syncthreads();
        if (wave < NS && active[wave]) {
            find_digit(hist[wave], krem[wave], lane, &sel_digit[wave], &sel_above[wave]);
        }
        __syncthreads();
        if (tid == 0) {
            for (int s = 0; s < NS; ++s) {
                if (!active[s]) continue;
                prefix[s] |= (uint64_t)sel_digit[s] << shift;
                krem[s] -= sel_above[s];
                if (hist[s][sel_digit[s]] == 1u) live[s] = 0;
            }
        }
        pmask |= (uint64_t)0xFFu << shift;
        __syncthreads();
    }

    uint64_t K[NS];
    bool all[NS], none[NS];
#pragma unroll
    for (int s = 0; s < NS; ++s) {
        K[s] = prefix[s];
        all[s] = ks[s] >= R;
        none[s] = ks[s] <= 0;
    }
    auto tier_of = [&](int64_t j, float sc) -> int {
        if (j < sinks) return 0;
        const uint64_t key = make_key(sc, j, bits);
        int tier = 3;
#pragma unroll
        for (int s = NS - 1; s >= 0; --s)
            if (!none[s] && (all[s] || key >= K[s])) tier = s;
        return tier;
    };
    const uint32_t base[4] = {0u, (uint32_t)n16, (uint32_t)(n16 + n8),
                              (uint32_t)(n16 + n8 + n4)};
    if (tid < 4) running[tid] = 0;
    __syncthreads();
    // Slots, kThreads * S tokens a round, S = kChunk steps or, in the last
    // round, as few as the remaining tokens need: wavefront w takes the
    // contiguous 64 * S tokens from t0 + 64 * S * w, 64 consecutive tokens a
    // step (coalesced).  A first walk finds every token's tier (2
    // bits per step, kept in one register) and the wavefront's count per
    // tier (ballots); one workgroup scan of those counts gives each
    // wavefront its offsets; a second walk numbers the tokens of each tier
    // in token order with ballot prefixes and writes map and order.
    const uint64_t below = (1ull << lane) - 1ull;  // lanes before this one
    for (int64_t t0 = 0; t0 < n;) {
        const int64_t left = n - t0;
        const int S = left >= (int64_t)kThreads * kChunk
                          ? kChunk
                          : (int)((left + kThreads - 1) / kThreads);
        const int64_t w0 = t0 + (int64_t)wave * 64 * S + lane;
        uint32_t packed = 0;
        uint32_t wc[4] = {0u, 0u, 0u, 0u};
        for (int b = 0; b < S; b += kBatch) {
            float sv[kBatch];
#pragma unroll
            for (int u = 0; u < kBatch; ++u) {
                const int64_t j = w0 + 64 * (b + u);
                sv[u] = (b + u < S && j < n) ? score[j] : 0.0f;
            }
#pragma unroll
            for (int u = 0; u < kBatch; ++u) {
                const int64_t j = w0 + 64 * (b + u);
                const int t = (b + u < S && j < n) ? tier_of(j, sv[u]) : 4;
                packed |= (uint32_t)(t & 3) << (2 * (b + u));
#pragma unroll
                for (int q = 0; q < 4; ++q) wc[q] += (uint32_t)__popcll(__ballot(t == q));
            }
        }
        if (lane < 4) wtot[wave][lane] = wc[lane];
        __syncthreads();
        uint32_t off[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            off[q] = running[q];
            for (int w = 0; w < wave; ++w) off[q] += wtot[w][q];
        }
        for (int i = 0; i < S; ++i) {
            const int64_t j = w0 + 64 * i;
            const bool valid = j < n;
            const int t = (int)((packed >> (2 * i)) & 3u);
            uint32_t slot = 0;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const unsigned long long bq = __ballot(valid && t == q);
                if (valid && t == q) slot = off[q] + (uint32_t)__popcll(bq & below);
                off[q] += (uint32_t)__popcll(bq);
            }
            if (valid) {
                map[j] = ((uint32_t)t << 30) | slot;
                order[base[t] + slot] = (uint32_t)j;
            }
        }
        __syncthreads();
        if (tid < 4) {
            uint32_t tot = 0;
            for (int w = 0; w < kWaves; ++w) tot += wtot[w][tid];
            running[tid] += tot;
        }
        __syncthreads();
        t0 += (int64_t)kThreads * S;
    }
}

// Balanced ranking key of the non-sink token at offset r = j - sinks:
// 2^b - 1 - bitreverse_b(r), b = fewest bits that hold R - 1 (exact in fp32
// for R <= 2^24); sinks get 0.
__global__ __launch_bounds__(256) void balanced_kernel(float* __restrict__ keys, int64_t n,
                                                       int64_t sinks, int b) {
    const int64_t j = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (j >= n) return;
    if (j < sinks) {
        keys[j] = 0.0f;
        return;
    }
    const uint32_t r = (uint32_t)(j - sinks);
    const uint32_t rev = b ? (__builtin_bitreverse32(r) >> (32 - b)) : 0u;
    keys[j] = (float)(((1u << b) - 1u) - rev);
}

}  // namespace

hipError_t launch_select(int64_t n, int64_t sinks, int64_t n16, int64_t n8, int64_t n4,
                         const float* score, uint32_t* map, uint32_t* order,
                         hipStream_t st) {
    const int64_t k1 = n16 - sinks;
    const int64_t k2 = k1 + n8;
    const int64_t k3 = k2 + n4;
    hipLaunchKernelGGL(select_kernel, dim3(1), dim3(kThreads), 0, st, score, n, sinks, k1, k2,
                       k3, n16, n8, n4, map, order);
    return hipGetLastError();
}

hipError_t launch_balanced(int64_t n, int64_t sinks, float* keys, hipStream_t st) {
    int b = 0;
    while (((int64_t)1 << b) < n - sinks) ++b;
    hipLaunchKernelGGL(balanced_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, keys,
                       n, sinks, b);
    return hipGetLastError();
}

}  // namespace sk
