/*
 * sk.h - C ABI of the per-token mixed-precision KV transfer path on MI355X.
 *
 * The operations follow the SpectrumKV paper (arXiv 2606.08635):
 *   - importance score            : §4.3 (I_j = A_j with lambda = 0) and
 *                                    Algorithm 1 "score tokens"; its recency
 *                                    weighting and KV-norm fallback
 *   - tier assignment             : §4.4 budget-to-tier mapping, §7.4.1 sink
 *                                    pinning, §2.3 Proposition 1 (sorted
 *                                    assignment), Algorithm 1 "assign tiers"
 *   - quantize + pack             : Algorithm 1 "transfer" (K and V quantized
 *                                    independently, one mixed payload), §2.1
 *                                    tier costs
 *   - dequantize (dense or paged) : §4.2 (decode-side dequantization only)
 *   - cold-tier upgrade           : §4.2 and §8 (cold-tier fetch design)
 *   - decode attention            : §4.2, from the payload without unpacking
 *
 * Conventions shared by every entry point
 *   - Ownership: the caller allocates and frees every buffer.  The library
 *     never allocates, frees or synchronizes, and keeps no pointer after a
 *     call returns.  It has no global mutable state except the per-thread
 *     error message and the static per-device scratch of sk_score_noalloc
 *     (with its looked-up addresses).
 *   - Streams: `stream` is a hipStream_t passed as void* (NULL = the null
 *     stream).  Device work is enqueued asynchronously on it.
 *   - Validation: all arguments are checked on the host before anything is
 *     enqueued.  On any error nothing is enqueued, no output is touched and a
 *     non-zero status is returned; sk_last_error() then describes it.
 *   - Device errors: a failed launch returns SK_E_DEVICE.  Faults inside a
 *     kernel surface at the caller's next synchronization.
 *   - Pointers to device memory must be 16-byte aligned; `payload` must be
 *     256-byte aligned.  All tensors are dense and row-major as documented.
 *   - Element types: fp16 = IEEE binary16, fp32 = IEEE binary32, little-endian.
 *   - n_tokens = 0 is a valid, empty request: every call returns SK_OK and
 *     enqueues nothing.
 */
#ifndef SK_H_
#define SK_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t sk_status;
#define SK_OK            0
#define SK_E_ARG         1  /* NULL / misaligned pointer, bad size, bad value */
#define SK_E_UNSUPPORTED 2  /* shape the kernels do not handle (head_dim, ...) */
#define SK_E_BUDGET      3  /* budget cannot pay every token at the cheapest tier */
#define SK_E_WORKSPACE   4  /* workspace smaller than the *_workspace_bytes query */
#define SK_E_DEVICE      5  /* a HIP launch failed */

#define SK_LAYOUT_V1 1
#define SK_TIER_FP16 0u
#define SK_TIER_INT8 1u
#define SK_TIER_INT4 2u
#define SK_TIER_DROP 3u   /* not sent (overflow mode SK_OVERFLOW_DROP) */
#define SK_MAP_TIER(m) ((uint32_t)(m) >> 30)
#define SK_MAP_SLOT(m) ((uint32_t)(m) & 0x3FFFFFFFu)

/* Model KV shape (§2.1: L layers, H_kv KV heads of dimension d_h; GQA query
 * head h reads KV head h / (n_q_heads / n_kv_heads)).
 * Supported: n_layers >= 1, n_kv_heads >= 1, n_q_heads a multiple of
 * n_kv_heads with n_q_heads / n_kv_heads <= 16, head_dim in {64, 128, 256}. */
typedef struct {
    int32_t n_layers;
    int32_t n_q_heads;
    int32_t n_kv_heads;
    int32_t head_dim;
} sk_shape;

/* What to do when the budget cannot pay every non-sink token at the
 * cheapest allowed tier (int4 in 3-tier, int8 in 2-tier):
 *   SK_OVERFLOW_REJECT   : sk_plan_make fails with SK_E_BUDGET (default)
 *   SK_OVERFLOW_DROP     : §7.4.3 (a 2-tier policy at b = 0.3 sends only 60%
 *                          of the tokens): floor(Br / cost) tokens are sent
 *                          at the cheapest tier and the lowest-ranked rest
 *                          are dropped (tier SK_TIER_DROP, no bytes); the
 *                          sinks must still fit (Br >= 0, else SK_E_BUDGET)
 *   SK_OVERFLOW_FALLBACK : the tier table of the Korean SpectrumKV summary
 *                          (lowest band int4 when allowed, else int8): every
 *                          token is sent at the cheapest tier, over budget */
#define SK_OVERFLOW_REJECT   0
#define SK_OVERFLOW_DROP     1
#define SK_OVERFLOW_FALLBACK 2

/* Transfer policy of one request.
 *   n_tokens   : n, 0 <= n < 2^30
 *   n_sink     : S >= 0, leading tokens pinned to fp16 (§7.4.1)
 *   three_tier : 1 = fp16/int8/int4 (int4 probe passed, §4.5), 0 = fp16/int8
 *   budget     : b in [0, 1], fraction of the fp16 bytes (§2.1, §4.4)
 *   overflow   : one of SK_OVERFLOW_* (zero-initialised policies reject) */
typedef struct {
    int64_t n_tokens;
    int32_t n_sink;
    int32_t three_tier;
    double  budget;
    int32_t overflow;
} sk_policy;

/* Tier counts and payload layout, a pure function of (shape, policy).
 *
 * Counts (§4.4 and §7.4.1; quarter-token units fp16 = 4, int8 = 2, int4 = 1):
 *   B  = floor(4 b n + 1e-7) evaluated in double,  S' = min(S, n),
 *   R  = n - S',  Br = B - 4 S'   (sinks are paid from the budget first)
 *   3-tier: Br < R -> SK_E_BUDGET;  Br <= 2R -> n16 = 0, n8 = Br - R,
 *           n4 = 2R - Br (the printed f8 = 4b-1, f4 = 2-4b); otherwise
 *           n16 = min(R, floor((Br - 2R)/2)), n8 = R - n16, n4 = 0.
 *   2-tier: Br < 2R -> SK_E_BUDGET; otherwise as the upper 3-tier branch.
 *   N16 = S' + n16, N8 = n8, N4 = n4.
 *   The SK_E_BUDGET cases above become, with overflow = SK_OVERFLOW_DROP,
 *   N4 (3-tier) or N8 (2-tier) = floor(Br / cost) and N_drop = R minus that,
 *   and with SK_OVERFLOW_FALLBACK, N4 or N8 = R (used_units > budget_units).
 *
 * Payload layout v1 (no padding): segments c16 | c8 | c4 | s8 | s4.
 *   A "row" is (layer l, slot, kv in {0 = K, 1 = V}, KV head g) of head_dim
 *   elements; within tier t its index is r = ((l * N_t + slot) * 2 + kv) * H + g.
 *   c16 : fp16 rows, 2d bytes each            (raw copy of the input)
 *   c8  : int8 two's complement codes, d bytes each
 *   c4  : int4 two's complement codes, d/2 bytes each, element 2m in bits
 *         0-3 and element 2m+1 in bits 4-7 of byte m
 *   s8, s4 : one fp16 scale per int8 / int4 row, same row order
 *   payload_bytes = L * 2H * (N16 * 2d + N8 * (d + 2) + N4 * (d/2 + 2)). */
typedef struct {
    int64_t n16, n8, n4;        /* n16 includes the sinks */
    int64_t n_drop;             /* tokens not sent: n = n16 + n8 + n4 + n_drop */
    int64_t n_sink;             /* S' */
    int64_t budget_units;       /* B */
    int64_t used_units;         /* 4 N16 + 2 N8 + N4 <= B */
    int64_t payload_bytes;
    int64_t off_c16, off_c8, off_c4, off_s8, off_s4;
    int64_t n_tokens;
    int32_t n_layers, n_kv_heads, head_dim, layout_version;
    uint64_t check;             /* hash of every field above; sk_pack and
                                   sk_unpack reject a plan whose hash or
                                   shape does not match */
} sk_plan;

/* Host only, pure, touches no device.  Returns SK_E_ARG / SK_E_UNSUPPORTED
 * for a bad shape or policy (SK_E_UNSUPPORTED too when the fp16 KV of the
 * request, 4 * L * n * H * d bytes, is beyond 2^62, so that every offset
 * fits int64) and SK_E_BUDGET when the budget cannot pay every token under
 * the policy's overflow mode (out is then left untouched). */
sk_status sk_plan_make(const sk_shape* shape, const sk_policy* policy, sk_plan* out);

/* ---------------------------------------------------------------- score --
 * Importance score of one layer (§4.3 with lambda = 0, Algorithm 1):
 *   A_j = sum_h sum_{i >= j} softmax_i(q_i . k_j / sqrt(d))_j,
 * the causal attention column sums of layer l over its H_q query heads.
 * Calling it once per layer with accumulate = (l > 0) yields
 * score_j = sum_l A_j (the attention received over all heads and layers).
 *
 *   q     : fp16 [n][n_q_heads][head_dim]  (this layer's post-RoPE queries)
 *   k     : fp16 [n][n_kv_heads][head_dim] (this layer's post-RoPE keys)
 *   score : fp32 [n]; overwritten (accumulate = 0) or added to (1)
 *   ws    : device workspace of at least sk_score_workspace_bytes(shape, n)
 *           bytes; its contents are scratch between calls.
 * Two passes run back to back on `stream`: a row log-sum-exp pass and a
 * column-sum pass that recomputes q.k with MFMA and sums exp(s - lse); the
 * per-query-head partial sums are then added in a fixed order, so the
 * result is deterministic.  The score calls (this one, sk_score_rowlse and
 * sk_score_colsum) take n_tokens <= 4,194,240 (65535 blocks of 64 queries);
 * a longer request returns SK_E_UNSUPPORTED, and the workspace queries
 * return 0 for it. */
size_t    sk_score_workspace_bytes(const sk_shape* shape, int64_t n_tokens);
sk_status sk_score(const sk_shape* shape, int64_t n_tokens,
                   const void* q, const void* k, float* score, int32_t accumulate,
                   void* ws, size_t ws_bytes, void* stream);

/* Allocation-free variant of sk_score, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc).  Same arguments, results and error behaviour as
 * sk_score, without the workspace: the lse values and per-head column sums
 * live in a static device array of SK_SCORE_SCRATCH_BYTES that the library
 * owns, one per GPU it runs on, held until the process ends (its address is
 * looked up on the first call on each device; a failed lookup returns
 * SK_E_DEVICE).  A request needing more than that
 * (sk_score_workspace_bytes(shape, n) > SK_SCORE_SCRATCH_BYTES, i.e. about
 * n_q_heads * n_tokens > 4.19M) returns SK_E_WORKSPACE before anything is
 * enqueued.  Nothing needs clearing between calls (every scratch byte a call
 * reads, that call wrote first), but all calls on one GPU share the array:
 * calls that overlap in time on one GPU (on different streams, or from
 * different host threads without ordering) race and give wrong results.
 * The call itself allocates and frees nothing. */
#define SK_SCORE_SCRATCH_BYTES ((size_t)32 << 20)
sk_status sk_score_noalloc(const sk_shape* shape, int64_t n_tokens,
                           const void* q, const void* k, float* score, int32_t accumulate,
                           void* stream);

/* The two passes of sk_score as separate calls (same results when chained).
 *   sk_score_rowlse : lse fp32 [n_q_heads][n], the base-2 logarithm of the
 *                     causal softmax denominator of row i of head h:
 *                     lse[h][i] = log2 sum_{j <= i} exp(q_i . k_j / sqrt(d))
 *                     (= the natural log-sum-exp times log2(e)); base 2 lets
 *                     the column pass weight each element with one exp2.
 *   sk_score_colsum : uses lse from sk_score_rowlse on the same q, k and
 *                     writes / accumulates score as sk_score does; ws must
 *                     hold sk_score_colsum_workspace_bytes(shape, n) bytes. */
sk_status sk_score_rowlse(const sk_shape* shape, int64_t n_tokens,
                          const void* q, const void* k, float* lse, void* stream);
size_t    sk_score_colsum_workspace_bytes(const sk_shape* shape, int64_t n_tokens);
sk_status sk_score_colsum(const sk_shape* shape, int64_t n_tokens,
                          const void* q, const void* k, const float* lse,
                          float* score, int32_t accumulate,
                          void* ws, size_t ws_bytes, void* stream);

/* All layers in one launch per pass: the importance score summed over the
 * layers (SpectrumKV paper §4.3 "Importance scores", Algorithm 1 "score
 * tokens"), the same as calling sk_score once per layer l = 0 .. n_layers - 1
 * with accumulate = (l > 0 || accumulate), bit for bit, for a caller that
 * holds every layer's queries and keys.  One launch per pass instead of one
 * per layer removes the per-launch fill and drain (about 30 us each), which
 * is a tenth of a layer's time at 8K tokens.  sk_score_colsum_layers takes
 * the lse that sk_score_rowlse_layers wrote for the same q and k.
 *   q     : fp16 [n_layers][n][n_q_heads][head_dim]
 *   k     : fp16 [n_layers][n][n_kv_heads][head_dim] (the layout sk_pack reads)
 *   score : fp32 [n]; overwritten (accumulate = 0) or added to (1)
 *   lse   : (sk_score_rowlse_layers) fp32 [n_layers][n_q_heads][n], each
 *           layer's lse as sk_score_rowlse writes it
 *   ws    : at least sk_score_layers_workspace_bytes (sk_score_layers) or
 *           sk_score_colsum_layers_workspace_bytes (sk_score_colsum_layers)
 *           bytes, n_layers times the one-layer sizes; scratch between calls.
 * Token limit and errors as sk_score; n_layers must be at most 65535.  A
 * shape whose all-layer workspace would not fit in size_t gets 0 from the
 * size queries and SK_E_UNSUPPORTED from the calls. */
size_t    sk_score_layers_workspace_bytes(const sk_shape* shape, int64_t n_tokens);
sk_status sk_score_layers(const sk_shape* shape, int64_t n_tokens,
                          const void* q, const void* k, float* score, int32_t accumulate,
                          void* ws, size_t ws_bytes, void* stream);
sk_status sk_score_rowlse_layers(const sk_shape* shape, int64_t n_tokens,
                                 const void* q, const void* k, float* lse, void* stream);
size_t    sk_score_colsum_layers_workspace_bytes(const sk_shape* shape, int64_t n_tokens);
sk_status sk_score_colsum_layers(const sk_shape* shape, int64_t n_tokens,
                                 const void* q, const void* k, const float* lse,
                                 float* score, int32_t accumulate,
                                 void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------- score variants --
 * The other two options of Algorithm 1 "score tokens".
 *
 * Recency weighting, the §4.3 importance formula I_j = A_j exp(-lambda Delta_j):
 *   score_out[j] = fp32_rn(score_in[j] * exp(-lambda * (n - 1 - j)))
 * evaluated in double precision.  The page defines neither Delta_j nor
 * lambda; Delta_j is read as the distance of token j from the last prefill
 * token, so lambda > 0 ranks recent tokens higher and lambda = 0 returns the
 * input unchanged.  Apply it once, after the last layer's sk_score.
 *   score_in, score_out : fp32 [n]; they may be the same buffer (in place)
 *   lambda              : finite and >= 0, else SK_E_ARG */
sk_status sk_recency_weight(int64_t n_tokens, double lambda, const float* score_in,
                            float* score_out, void* stream);

/* KV-norm fallback (Algorithm 1 "score tokens"): a score that needs no
 * queries.  The page names it without a formula; it is read as the sum of the
 * Euclidean norms of the token's keys over layers and KV heads:
 *   score_j = sum_l sum_g || k[l][j][g][:] ||_2
 *   k     : fp16 [n_layers][n][n_kv_heads][head_dim] (the layout sk_pack
 *           reads; a caller holding one buffer per layer passes
 *           n_layers = 1 and accumulates)
 *   score : fp32 [n]; overwritten (accumulate = 0) or added to (1)
 * Sums of squares, square roots and the sum over (l, g) are fp32 in a fixed
 * order, so the result is deterministic; its relative error is at most
 * (m + 16) * 2^-24 with m = ceil(n_layers * ceil(n_kv_heads * head_dim / 512) / 8)
 * (2e-6 for 32 layers x 8 heads x 128). */
sk_status sk_score_kvnorm(const sk_shape* shape, int64_t n_tokens, const void* k,
                          float* score, int32_t accumulate, void* stream);

/* --------------------------------------------------------------- assign --
 * Tier assignment (§7.4.1 sinks, §2.3 sorted assignment, §4.4 counts):
 * tokens j < S' get fp16; the others are ranked by (score descending, token
 * index ascending) - ties go to the lower index - and the first n16 - S'
 * take fp16, the next n8 int8, the next n4 int4 and the rest (n_drop) are
 * dropped (SK_TIER_DROP; pack and unpack skip them).
 *
 * Assignment-only variants (§7 baselines, §7.4.1 Table 11, §7.4.2 Table 12)
 * rank by another key passed as `score`: Random_Tier keeps the tier counts
 * and ranks by caller-drawn i.i.d. random keys; Balanced ranks by the keys
 * of sk_balanced_keys, which spread every tier evenly over the positions
 * regardless of importance.
 *   score : fp32 [n], finite and >= 0 (-0.0 counts as +0.0; NaN/Inf: the
 *           output is unspecified but every write stays in bounds)
 *   map   : u32 [n], map[j] = tier << 30 | slot, slot = number of tokens
 *           j' < j with the same tier
 *   order : u32 [n], the tokens sorted by (tier, index): fp16 slots first,
 *           then int8, then int4, then dropped; order[off_t + slot] = j
 *   ws    : at least sk_assign_workspace_bytes(n) bytes. */
size_t    sk_assign_workspace_bytes(int64_t n_tokens);
/* Balanced keys: keys[j] = 0 for j < S' = min(n_sink, n); for the others,
 * with r = j - S', R = n - S' and b the fewest bits that hold R - 1,
 * keys[j] = 2^b - 1 - bitreverse_b(r) (fp32, exact): ranking by it visits
 * the positions in van der Corput order, so the tokens of every tier are
 * spread evenly over the sequence.  R > 2^24 -> SK_E_UNSUPPORTED. */
sk_status sk_balanced_keys(int64_t n_tokens, int32_t n_sink, float* keys, void* stream);
sk_status sk_assign_tiers(const sk_policy* policy, const sk_plan* plan,
                          const float* score, uint32_t* map, uint32_t* order,
                          void* ws, size_t ws_bytes, void* stream);

/* ----------------------------------------------------------------- pack --
 * Quantize + compact (Algorithm 1 "transfer").  Per row of d elements:
 * fp16 rows are copied; int8 / int4 rows use a symmetric absmax scale
 *   s = fp16_rne(fl32(max|x| / qmax)),  qmax = 127 / 7,
 *   q = clamp(rint_even(fl32(x / s)), -qmax, qmax)   (q = 0 when s == 0),
 * written at the row's slot in the layout described at sk_plan.
 *   k, v    : fp16 [n_layers][n][n_kv_heads][head_dim], finite (a NaN or
 *             Inf in an int8 / int4 row leaves that row's codes and scale
 *             unspecified; every write stays in bounds)
 *   map     : from sk_assign_tiers (entries whose slot is out of range for
 *             their tier are skipped)
 *   order   : from sk_assign_tiers (may be NULL; reserved for layouts that
 *             need it)
 *   payload : plan->payload_bytes bytes, 256-byte aligned; every byte is
 *             written when map is a valid assignment. */
sk_status sk_pack(const sk_shape* shape, const sk_plan* plan,
                  const void* k, const void* v,
                  const uint32_t* map, const uint32_t* order,
                  void* payload, void* stream);

/* --------------------------------------------------------------- unpack --
 * Decode side (§4.2): x_hat = fp16_rne(float(q) * float(s)) for int rows,
 * the raw fp16 row otherwise.
 * Dense:  paged == NULL, k_out / v_out fp16 [n_layers][n][n_kv_heads][head_dim]
 *         (every element written, except the rows of dropped tokens, which
 *         are left untouched; attention must mask those tokens out).
 * Paged:  k_out = v_out = NULL; token j of layer l is written to
 *         cache[l][block_table[j / block_size]][j % block_size][g][:] of
 *         k_cache and v_cache, both fp16
 *         [n_layers][num_blocks][block_size][n_kv_heads][head_dim].  Rows of
 *         blocks that hold no token of this request are untouched; a token
 *         whose block id lies outside [0, num_blocks) is skipped. */
typedef struct {
    void* k_cache;
    void* v_cache;
    const int32_t* block_table;   /* device, [ceil(n / block_size)] */
    int32_t block_size;           /* >= 1 */
    int64_t num_blocks;           /* >= ceil(n / block_size) */
} sk_paged;

sk_status sk_unpack(const sk_shape* shape, const sk_plan* plan,
                    const void* payload, const uint32_t* map,
                    void* k_out, void* v_out, const sk_paged* paged, void* stream);

/* -------------------------------------------------------------- upgrade --
 * Cold-tier upgrade (§4.2, and the cold-tier fetch design paragraph of §8):
 * tokens that reached the decode side at int8 or int4 are raised to fp16
 * later by re-sending their fp16 rows, which then overwrite the
 * approximations in the decode-side KV.  The pages give the saving only as a
 * byte difference; no code shorter than 16 bits per element restores every
 * fp16 value from its int4 bucket, so the rows are sent whole.
 *   tokens  : device u32 [n_up], token indices chosen by the caller; an entry
 *             >= n_tokens is skipped (its payload rows are not written and
 *             nothing is written for it on unpack); repeats are allowed
 *   payload : sk_upgrade_bytes(shape, n_up) bytes, 16-byte aligned; row
 *             r = ((l * n_up + i) * 2 + kv) * n_kv_heads + g holds the fp16
 *             row of token tokens[i] (the c16 layout of sk_plan with
 *             N16 = n_up and slot = i), 2 * head_dim bytes each.
 * sk_upgrade_pack reads k, v as sk_pack does.  sk_upgrade_unpack writes the
 * rows into dense k_out / v_out (paged == NULL) or into the paged cache
 * exactly where sk_unpack puts the token (a block id outside the pool is
 * skipped); all other rows are untouched.
 * sk_upgrade_bytes returns 0 for an invalid shape or n_up < 0. */
size_t    sk_upgrade_bytes(const sk_shape* shape, int64_t n_up);
sk_status sk_upgrade_pack(const sk_shape* shape, int64_t n_tokens, const void* k,
                          const void* v, const uint32_t* tokens, int64_t n_up,
                          void* payload, void* stream);
sk_status sk_upgrade_unpack(const sk_shape* shape, int64_t n_tokens, const void* payload,
                            const uint32_t* tokens, int64_t n_up, void* k_out, void* v_out,
                            const sk_paged* paged, void* stream);

/* --------------------------------------------------------------- decode --
 * Decode attention straight from the payload (§4.2: the decode worker
 * dequantizes and runs attention; here the dequantization happens while the
 * payload is read, with no dense KV).  For every layer l in
 * [layer0, layer0 + n_layers_q) and query head h (KV head g = h / (H_q/H_kv)):
 *   o[l][h]   = sum_j softmax_j(q[l][h] . k_hat_j / sqrt(d)) v_hat_j
 *   lse[l][h] = ln sum_j exp(q[l][h] . k_hat_j / sqrt(d))
 * over the tokens that were sent (dropped tokens take no part; no causal
 * mask: a decode query follows the whole prefix), where k_hat, v_hat are
 * exactly the fp16 rows sk_unpack would write.  The decode step's own new
 * token is not included: merge it with the returned lse.  With no token
 * sent, o = 0 and lse = -inf.
 *   q       : fp16 [n_layers_q][n_q_heads][head_dim], 16-byte aligned
 *   out     : fp32 [n_layers_q][n_q_heads][head_dim]
 *   lse     : fp32 [n_layers_q][n_q_heads] (natural log) or NULL
 *   payload : as written by sk_pack for `plan` (256-byte aligned)
 *   ws      : at least sk_decode_workspace_bytes(shape, plan, n_layers_q)
 * Arithmetic: q.k and p.v in fp32 from packed fp16 products; probabilities
 * are rounded to fp16 once (used in both the numerator and the
 * denominator), so o is a convex combination of the v_hat rows within
 * about 1e-3 * max|v_hat| of the exact value.  Deterministic.
 * Shapes with more than 65535 KV heads (a launch grid dimension) get 0 from
 * the workspace query and SK_E_UNSUPPORTED from the call. */
size_t    sk_decode_workspace_bytes(const sk_shape* shape, const sk_plan* plan,
                                    int32_t n_layers_q);
sk_status sk_decode_attention(const sk_shape* shape, const sk_plan* plan, const void* payload,
                              int32_t layer0, int32_t n_layers_q, const void* q, float* out,
                              float* lse, void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------ messages -- */
const char* sk_status_string(sk_status status);
/* Message of the last failing call on this thread ("" if none). */
const char* sk_last_error(void);
/* Layout version implemented (SK_LAYOUT_V1). */
int32_t sk_layout_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SK_H_ */
