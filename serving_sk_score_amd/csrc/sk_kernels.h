// Internal launchers of the HIP kernels behind include/sk.h.  Every launcher
// assumes its arguments were validated by the C-ABI layer (sk_api.cpp) and
// only enqueues work on `stream`.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sk {

struct Dims {
    int32_t L, Hq, Hkv, d;
    int64_t n;
};

// Layout of one tier's rows inside the payload.
struct TierSeg {
    int64_t count;     // N_t
    int64_t off_code;  // byte offset of the code segment
    int64_t off_scale; // byte offset of the scale segment (int tiers)
};

// score pass 1: lse fp32 [Hq][n], base-2 log of the causal softmax
// denominator; with layers > 1, q [layers][n][Hq][d], k [layers][n][Hkv][d]
// and lse [layers][Hq][n], all layers in one launch
hipError_t launch_rowlse(const Dims& s, const void* q, const void* k, float* lse,
                         hipStream_t st, int layers = 1);
// score pass 2: per-query-head column sums, partial fp32 [Hq][n_pad],
// n_pad = padded_tokens(n) (with layers > 1: [layers][Hq][n_pad])
hipError_t launch_colsum(const Dims& s, const void* q, const void* k, const float* lse,
                         float* partial, hipStream_t st, int layers = 1);
// score[j] = (acc ? score[j] : 0) + sum_h partial[h][j], h in order
hipError_t launch_reduce(const Dims& s, const float* partial, float* score, int acc,
                         hipStream_t st);
// the same for each of `layers` partial blocks in layer order, as one call of
// launch_reduce per layer (accumulating from the second on) would; row 0 of
// each layer's block is overwritten with that layer's head sum
hipError_t launch_reduce_layers(const Dims& s, float* partial, float* score, int acc,
                                hipStream_t st, int layers);
int64_t padded_tokens(int64_t n);
// Device address and size of the static score workspace on the current
// device (looked up once per device).
hipError_t score_scratch(void** ptr, size_t* bytes);
// number of rows of the pass-2 partial buffer
int colsum_partial_rows(const Dims& s);

// Balanced-variant ranking keys (fp32 [n], n - sinks <= 2^24)
hipError_t launch_balanced(int64_t n, int64_t sinks, float* keys, hipStream_t st);

// tier selection (n16 + n8 + n4 <= n; the lowest-ranked rest get tier 3)
hipError_t launch_select(int64_t n, int64_t sinks, int64_t n16, int64_t n8, int64_t n4,
                         const float* score, uint32_t* map, uint32_t* order,
                         hipStream_t st);

// pack / unpack
hipError_t launch_pack(const Dims& s, const TierSeg seg[3], const void* k, const void* v,
                       const uint32_t* map, void* payload, hipStream_t st);
hipError_t launch_unpack_dense(const Dims& s, const TierSeg seg[3], const void* payload,
                               const uint32_t* map, void* k_out, void* v_out,
                               hipStream_t st);
hipError_t launch_unpack_paged(const Dims& s, const TierSeg seg[3], const void* payload,
                               const uint32_t* map, void* k_cache, void* v_cache,
                               const int32_t* block_table, int32_t block_size,
                               int64_t num_blocks, hipStream_t st);

// cold-tier upgrade: fp16 rows of m listed tokens (block_table NULL = dense)
hipError_t launch_upgrade_pack(const Dims& s, int64_t m, const void* k, const void* v,
                               const uint32_t* tokens, void* payload, hipStream_t st);
hipError_t launch_upgrade_unpack(const Dims& s, int64_t m, const void* payload,
                                 const uint32_t* tokens, void* k_out, void* v_out,
                                 const int32_t* block_table, int32_t block_size,
                                 int64_t num_blocks, hipStream_t st);

// decode attention from the payload: partial records fp32
// [nl][Hq][decode_chunks][d + 2], then out fp32 [nl][Hq][d] and lse fp32 [nl][Hq]
int decode_tiles_per_chunk(const Dims& s, const TierSeg seg[3], int nl);
int64_t decode_chunks(const Dims& s, const TierSeg seg[3], int nl);
hipError_t launch_decode(const Dims& s, const TierSeg seg[3], const void* payload, int layer0,
                         int nl, const void* q, float* out, float* lse, float* part,
                         hipStream_t st);

// score variants: KV-norm fallback (score fp32 [n]) and recency weighting
hipError_t launch_kvnorm(const Dims& s, const void* k, float* score, int accumulate,
                         hipStream_t st);
hipError_t launch_recency(int64_t n, double lambda, const float* in, float* out,
                          hipStream_t st);

}  // namespace sk
