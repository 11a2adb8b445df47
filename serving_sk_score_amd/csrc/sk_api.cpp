// C-ABI layer: argument validation, the tier-count / layout closed form and
// dispatch to the HIP kernels.  Nothing is enqueued unless every check passes.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>

#include "../../include/sk.h"
#include "sk_kernels.h"

namespace {

thread_local std::string g_err;

sk_status fail(sk_status st, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_err = buf;
    return st;
}

sk_status ok() {
    g_err.clear();
    return SK_OK;
}

constexpr int64_t kMaxTokens = (int64_t)1 << 30;

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

sk_status check_shape(const sk_shape* s) {
    if (!s) return fail(SK_E_ARG, "shape is NULL");
    if (s->n_layers < 1 || s->n_q_heads < 1 || s->n_kv_heads < 1)
        return fail(SK_E_ARG, "shape: n_layers, n_q_heads and n_kv_heads must be >= 1");
    if (s->n_q_heads % s->n_kv_heads)
        return fail(SK_E_ARG, "shape: n_q_heads (%d) is not a multiple of n_kv_heads (%d)",
                    s->n_q_heads, s->n_kv_heads);
    if (s->n_q_heads / s->n_kv_heads > 16)
        return fail(SK_E_UNSUPPORTED, "shape: more than 16 query heads per KV head");
    if (s->head_dim != 64 && s->head_dim != 128 && s->head_dim != 256)
        return fail(SK_E_UNSUPPORTED, "shape: head_dim %d not in {64, 128, 256}", s->head_dim);
    if (s->n_layers > 65535) return fail(SK_E_UNSUPPORTED, "shape: more than 65535 layers");
    return SK_OK;
}

// Whether the fp16 K and V of n tokens, 4 * L * n * H * d bytes, stay within
// 2^62: then every payload offset and size (at most twice that) fits int64.
bool kv_fits(const sk_shape* s, int64_t n) {
    const __int128 kv = (__int128)4 * s->n_layers * n * s->n_kv_heads * s->head_dim;
    return kv <= ((__int128)1 << 62);
}

sk_status check_tokens(int64_t n) {
    if (n < 0 || n >= kMaxTokens) return fail(SK_E_ARG, "n_tokens %lld outside [0, 2^30)", (long long)n);
    return SK_OK;
}

uint64_t plan_hash(const sk_plan& p) {
    const int64_t f[] = {p.n16, p.n8, p.n4, p.n_drop, p.n_sink, p.budget_units, p.used_units,
                         p.payload_bytes, p.off_c16, p.off_c8, p.off_c4, p.off_s8, p.off_s4,
                         p.n_tokens, p.n_layers, p.n_kv_heads, p.head_dim, p.layout_version};
    uint64_t h = 1469598103934665603ull;  // FNV-1a
    for (int64_t v : f) {
        for (int b = 0; b < 8; ++b) {
            h ^= (uint64_t)((v >> (8 * b)) & 0xFF);
            h *= 1099511628211ull;
        }
    }
    return h;
}

sk_status check_plan(const sk_plan* p, const sk_shape* s) {
    if (!p) return fail(SK_E_ARG, "plan is NULL");
    if (p->layout_version != SK_LAYOUT_V1) return fail(SK_E_ARG, "plan: unknown layout version");
    if (p->check != plan_hash(*p)) return fail(SK_E_ARG, "plan: checksum mismatch (corrupted plan)");
    if (s && (p->n_layers != s->n_layers || p->n_kv_heads != s->n_kv_heads ||
              p->head_dim != s->head_dim))
        return fail(SK_E_ARG, "plan was made for a different shape");
    return SK_OK;
}

sk::Dims dims(const sk_shape* s, int64_t n) {
    return sk::Dims{s->n_layers, s->n_q_heads, s->n_kv_heads, s->head_dim, n};
}

void segs(const sk_plan* p, sk::TierSeg seg[3]) {
    seg[0] = {p->n16, p->off_c16, 0};
    seg[1] = {p->n8, p->off_c8, p->off_s8};
    seg[2] = {p->n4, p->off_c4, p->off_s4};
}

sk_status device(hipError_t e, const char* what) {
    if (e != hipSuccess) return fail(SK_E_DEVICE, "%s: %s", what, hipGetErrorString(e));
    return ok();
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

size_t lse_bytes(const sk_shape* s, int64_t n) {
    return align256((size_t)s->n_q_heads * (size_t)n * sizeof(float));
}

size_t partial_bytes(const sk_shape* s, int64_t n) {
    const sk::Dims d = dims(s, n);
    return align256((size_t)sk::colsum_partial_rows(d) * (size_t)sk::padded_tokens(n) *
                    sizeof(float));
}

}  // namespace

extern "C" {

int32_t sk_layout_version(void) { return SK_LAYOUT_V1; }

const char* sk_status_string(sk_status st) {
    switch (st) {
        case SK_OK: return "SK_OK";
        case SK_E_ARG: return "SK_E_ARG: invalid argument";
        case SK_E_UNSUPPORTED: return "SK_E_UNSUPPORTED: unsupported shape";
        case SK_E_BUDGET: return "SK_E_BUDGET: budget cannot pay every token";
        case SK_E_WORKSPACE: return "SK_E_WORKSPACE: workspace too small";
        case SK_E_DEVICE: return "SK_E_DEVICE: HIP launch failed";
        default: return "unknown sk_status";
    }
}

const char* sk_last_error(void) { return g_err.c_str(); }

sk_status sk_plan_make(const sk_shape* shape, const sk_policy* pol, sk_plan* out) {
    if (sk_status st = check_shape(shape)) return st;
    if (!pol || !out) return fail(SK_E_ARG, "policy and out must be non-NULL");
    if (sk_status st = check_tokens(pol->n_tokens)) return st;
    if (pol->n_sink < 0) return fail(SK_E_ARG, "n_sink must be >= 0");
    if (pol->three_tier != 0 && pol->three_tier != 1)
        return fail(SK_E_ARG, "three_tier must be 0 or 1");
    if (!std::isfinite(pol->budget) || pol->budget < 0.0 || pol->budget > 1.0)
        return fail(SK_E_ARG, "budget must be a finite fraction in [0, 1]");
    if (pol->overflow != SK_OVERFLOW_REJECT && pol->overflow != SK_OVERFLOW_DROP &&
        pol->overflow != SK_OVERFLOW_FALLBACK)
        return fail(SK_E_ARG, "overflow must be one of SK_OVERFLOW_*");
    if (!kv_fits(shape, pol->n_tokens))
        return fail(SK_E_UNSUPPORTED, "shape: the fp16 KV of %lld tokens is beyond 2^62 bytes",
                    (long long)pol->n_tokens);

    const int64_t n = pol->n_tokens;
    const int64_t S = pol->n_sink < n ? pol->n_sink : n;
    const int64_t R = n - S;
    // quarter-token units: fp16 = 4, int8 = 2, int4 = 1
    const int64_t B = (int64_t)std::floor(4.0 * pol->budget * (double)n + 1e-7);
    const int64_t Br = B - 4 * S;
    int64_t n16 = 0, n8 = 0, n4 = 0;
    const int64_t cheapest = pol->three_tier ? 1 : 2;  // units of the cheapest tier
    if (Br < cheapest * R && pol->overflow != SK_OVERFLOW_REJECT) {
        int64_t kept = R;
        if (pol->overflow == SK_OVERFLOW_DROP) {
            if (Br < 0)
                return fail(SK_E_BUDGET, "budget %.6g does not pay the %lld sinks", pol->budget,
                            (long long)S);
            kept = Br / cheapest;
        }
        (pol->three_tier ? n4 : n8) = kept;
    } else if (pol->three_tier) {
        if (Br < R)
            return fail(SK_E_BUDGET, "budget %.6g pays %lld quarter units for %lld tokens",
                        pol->budget, (long long)Br, (long long)R);
        if (Br <= 2 * R) {
            n8 = Br - R;
            n4 = 2 * R - Br;
        } else {
            n16 = (Br - 2 * R) / 2;
            if (n16 > R) n16 = R;
            n8 = R - n16;
        }
    } else {
        if (Br < 2 * R)
            return fail(SK_E_BUDGET, "2-tier budget %.6g pays %lld quarter units for %lld tokens",
                        pol->budget, (long long)Br, (long long)R);
        n16 = (Br - 2 * R) / 2;
        if (n16 > R) n16 = R;
        n8 = R - n16;
    }
    sk_plan p;
    std::memset(&p, 0, sizeof(p));
    p.n16 = S + n16;
    p.n8 = n8;
    p.n4 = n4;
    p.n_drop = R - n16 - n8 - n4;
    p.n_sink = S;
    p.budget_units = B;
    p.used_units = 4 * p.n16 + 2 * p.n8 + p.n4;
    const int64_t L = shape->n_layers, H = shape->n_kv_heads, d = shape->head_dim;
    const int64_t rows16 = L * p.n16 * 2 * H, rows8 = L * p.n8 * 2 * H, rows4 = L * p.n4 * 2 * H;
    p.off_c16 = 0;
    p.off_c8 = p.off_c16 + rows16 * 2 * d;
    p.off_c4 = p.off_c8 + rows8 * d;
    p.off_s8 = p.off_c4 + rows4 * (d / 2);
    p.off_s4 = p.off_s8 + rows8 * 2;
    p.payload_bytes = p.off_s4 + rows4 * 2;
    p.n_tokens = n;
    p.n_layers = shape->n_layers;
    p.n_kv_heads = shape->n_kv_heads;
    p.head_dim = shape->head_dim;
    p.layout_version = SK_LAYOUT_V1;
    p.check = plan_hash(p);
    *out = p;
    return ok();
}

// The row pass launches one workgroup row per 64 queries (for four heads per
// workgroup) and a launch grid holds at most 65535 rows.
constexpr int64_t kMaxScoreTokens = (int64_t)65535 * 64;

size_t sk_score_colsum_workspace_bytes(const sk_shape* shape, int64_t n) {
    if (check_shape(shape) || check_tokens(n) || n > kMaxScoreTokens) return 0;
    return partial_bytes(shape, n);
}

size_t sk_score_workspace_bytes(const sk_shape* shape, int64_t n) {
    if (check_shape(shape) || check_tokens(n) || n > kMaxScoreTokens) return 0;
    return lse_bytes(shape, n) + partial_bytes(shape, n);
}

static sk_status check_score_io(const sk_shape* shape, int64_t n, const void* q, const void* k) {
    if (sk_status st = check_shape(shape)) return st;
    if (sk_status st = check_tokens(n)) return st;
    if (n > kMaxScoreTokens)
        return fail(SK_E_UNSUPPORTED, "score: n_tokens %lld above %lld", (long long)n,
                    (long long)kMaxScoreTokens);
    if (n > 0 && (!q || !k)) return fail(SK_E_ARG, "q and k must be non-NULL");
    if (!aligned(q, 16) || !aligned(k, 16)) return fail(SK_E_ARG, "q and k must be 16-byte aligned");
    return SK_OK;
}

sk_status sk_score_rowlse(const sk_shape* shape, int64_t n, const void* q, const void* k,
                          float* lse, void* stream) {
    if (sk_status st = check_score_io(shape, n, q, k)) return st;
    if (n > 0 && !lse) return fail(SK_E_ARG, "lse must be non-NULL");
    if (!aligned(lse, 4)) return fail(SK_E_ARG, "lse must be 4-byte aligned");
    if (n == 0) return ok();
    (void)hipGetLastError();
    return device(sk::launch_rowlse(dims(shape, n), q, k, lse, (hipStream_t)stream), "rowlse");
}

sk_status sk_score_colsum(const sk_shape* shape, int64_t n, const void* q, const void* k,
                          const float* lse, float* score, int32_t accumulate, void* ws,
                          size_t ws_bytes, void* stream) {
    if (sk_status st = check_score_io(shape, n, q, k)) return st;
    if (n > 0 && (!lse || !score)) return fail(SK_E_ARG, "lse and score must be non-NULL");
    if (!aligned(lse, 4) || !aligned(score, 4)) return fail(SK_E_ARG, "lse and score must be 4-byte aligned");
    if (accumulate != 0 && accumulate != 1) return fail(SK_E_ARG, "accumulate must be 0 or 1");
    if (n == 0) return ok();
    const size_t need = partial_bytes(shape, n);
    if (!ws || ws_bytes < need)
        return fail(SK_E_WORKSPACE, "colsum workspace needs %zu bytes, got %zu", need, ws_bytes);
    if (!aligned(ws, 16)) return fail(SK_E_ARG, "workspace must be 16-byte aligned");
    const sk::Dims d = dims(shape, n);
    (void)hipGetLastError();
    hipError_t e = sk::launch_colsum(d, q, k, lse, (float*)ws, (hipStream_t)stream);
    if (e != hipSuccess) return device(e, "colsum");
    return device(sk::launch_reduce(d, (const float*)ws, score, accumulate, (hipStream_t)stream),
                  "reduce");
}

// ---- all layers per launch

// n_layers times a one-layer workspace size, or 0 when the product does not
// fit in size_t (a shape no device could hold; the calls then refuse it)
static size_t times_layers(const sk_shape* shape, size_t per_layer) {
    size_t r;
    if (__builtin_mul_overflow((size_t)shape->n_layers, per_layer, &r)) return 0;
    return r;
}

size_t sk_score_colsum_layers_workspace_bytes(const sk_shape* shape, int64_t n) {
    if (check_shape(shape) || check_tokens(n) || n > kMaxScoreTokens) return 0;
    return times_layers(shape, partial_bytes(shape, n));
}

size_t sk_score_layers_workspace_bytes(const sk_shape* shape, int64_t n) {
    if (check_shape(shape) || check_tokens(n) || n > kMaxScoreTokens) return 0;
    return times_layers(shape, lse_bytes(shape, n) + partial_bytes(shape, n));
}

sk_status sk_score_rowlse_layers(const sk_shape* shape, int64_t n, const void* q,
                                 const void* k, float* lse, void* stream) {
    if (sk_status st = check_score_io(shape, n, q, k)) return st;
    if (n > 0 && !lse) return fail(SK_E_ARG, "lse must be non-NULL");
    if (!aligned(lse, 4)) return fail(SK_E_ARG, "lse must be 4-byte aligned");
    if (n == 0) return ok();
    (void)hipGetLastError();
    return device(sk::launch_rowlse(dims(shape, n), q, k, lse, (hipStream_t)stream,
                                    shape->n_layers),
                  "rowlse");
}

// lse [L][Hq][n] (dense per layer) -> partial [L][Hq][n_pad] -> score
static sk_status run_colsum_layers(const sk_shape* shape, int64_t n, const void* q,
                                   const void* k, const float* lse, float* score,
                                   int32_t accumulate, float* partial, hipStream_t st) {
    const sk::Dims d = dims(shape, n);
    hipError_t e = sk::launch_colsum(d, q, k, lse, partial, st, shape->n_layers);
    if (e != hipSuccess) return device(e, "colsum");
    return device(sk::launch_reduce_layers(d, partial, score, accumulate, st, shape->n_layers),
                  "reduce");
}

sk_status sk_score_colsum_layers(const sk_shape* shape, int64_t n, const void* q,
                                 const void* k, const float* lse, float* score,
                                 int32_t accumulate, void* ws, size_t ws_bytes, void* stream) {
    if (sk_status st = check_score_io(shape, n, q, k)) return st;
    if (n > 0 && (!lse || !score)) return fail(SK_E_ARG, "lse and score must be non-NULL");
    if (!aligned(lse, 4) || !aligned(score, 4)) return fail(SK_E_ARG, "lse and score must be 4-byte aligned");
    if (accumulate != 0 && accumulate != 1) return fail(SK_E_ARG, "accumulate must be 0 or 1");
    if (n == 0) return ok();
    const size_t need = sk_score_colsum_layers_workspace_bytes(shape, n);
    if (need == 0) return fail(SK_E_UNSUPPORTED, "colsum workspace size overflows size_t");
    if (!ws || ws_bytes < need)
        return fail(SK_E_WORKSPACE, "colsum workspace needs %zu bytes, got %zu", need, ws_bytes);
    if (!aligned(ws, 16)) return fail(SK_E_ARG, "workspace must be 16-byte aligned");
    (void)hipGetLastError();
    return run_colsum_layers(shape, n, q, k, lse, score, accumulate, (float*)ws,
                             (hipStream_t)stream);
}

static sk_status check_score_call(const sk_shape* shape, int64_t n, const void* q,
                                   const void* k, const float* score, int32_t accumulate) {
    if (sk_status st = check_score_io(shape, n, q, k)) return st;
    if (n > 0 && !score) return fail(SK_E_ARG, "score must be non-NULL");
    if (!aligned(score, 4)) return fail(SK_E_ARG, "score must be 4-byte aligned");
    if (accumulate != 0 && accumulate != 1) return fail(SK_E_ARG, "accumulate must be 0 or 1");
    return SK_OK;
}

// The three launches of a score call over a validated workspace of
// lse_bytes + partial_bytes bytes.
static sk_status run_score(const sk_shape* shape, int64_t n, const void* q, const void* k,
                           float* score, int32_t accumulate, void* ws, void* stream) {
    const sk::Dims d = dims(shape, n);
    float* lse = (float*)ws;
    float* partial = (float*)((char*)ws + lse_bytes(shape, n));
    hipStream_t st = (hipStream_t)stream;
    (void)hipGetLastError();
    hipError_t e = sk::launch_rowlse(d, q, k, lse, st);
    if (e != hipSuccess) return device(e, "rowlse");
    e = sk::launch_colsum(d, q, k, lse, partial, st);
    if (e != hipSuccess) return device(e, "colsum");
    return device(sk::launch_reduce(d, partial, score, accumulate, st), "reduce");
}

sk_status sk_score(const sk_shape* shape, int64_t n, const void* q, const void* k, float* score,
                   int32_t accumulate, void* ws, size_t ws_bytes, void* stream) {
    if (sk_status st = check_score_call(shape, n, q, k, score, accumulate)) return st;
    if (n == 0) return ok();
    const size_t need = lse_bytes(shape, n) + partial_bytes(shape, n);
    if (!ws || ws_bytes < need)
        return fail(SK_E_WORKSPACE, "score workspace needs %zu bytes, got %zu", need, ws_bytes);
    if (!aligned(ws, 16)) return fail(SK_E_ARG, "workspace must be 16-byte aligned");
    return run_score(shape, n, q, k, score, accumulate, ws, stream);
}

sk_status sk_score_noalloc(const sk_shape* shape, int64_t n, const void* q, const void* k,
                           float* score, int32_t accumulate, void* stream) {
    if (sk_status st = check_score_call(shape, n, q, k, score, accumulate)) return st;
    if (n == 0) return ok();
    const size_t need = lse_bytes(shape, n) + partial_bytes(shape, n);
    if (need > SK_SCORE_SCRATCH_BYTES)
        return fail(SK_E_WORKSPACE,
                    "sk_score_noalloc: n_q_heads %d x n_tokens %lld needs %zu scratch bytes, "
                    "the static scratch holds %zu; use sk_score with a workspace",
                    shape->n_q_heads, (long long)n, need, (size_t)SK_SCORE_SCRATCH_BYTES);
    void* ws = nullptr;
    size_t have = 0;
    hipError_t e = sk::score_scratch(&ws, &have);
    if (e != hipSuccess) return device(e, "score scratch lookup");
    if (have < need) return fail(SK_E_WORKSPACE, "score scratch holds %zu bytes", have);
    return run_score(shape, n, q, k, score, accumulate, ws, stream);
}

sk_status sk_score_layers(const sk_shape* shape, int64_t n, const void* q, const void* k,
                          float* score, int32_t accumulate, void* ws, size_t ws_bytes,
                          void* stream) {
    if (sk_status st = check_score_call(shape, n, q, k, score, accumulate)) return st;
    if (n == 0) return ok();
    const size_t need = sk_score_layers_workspace_bytes(shape, n);
    if (need == 0) return fail(SK_E_UNSUPPORTED, "score workspace size overflows size_t");
    if (!ws || ws_bytes < need)
        return fail(SK_E_WORKSPACE, "score workspace needs %zu bytes, got %zu", need, ws_bytes);
    if (!aligned(ws, 16)) return fail(SK_E_ARG, "workspace must be 16-byte aligned");
    // lse [L][Hq][n] (dense), then the partials from an aligned offset
    float* lse = (float*)ws;
    float* partial = (float*)((char*)ws + (size_t)shape->n_layers * lse_bytes(shape, n));
    hipStream_t st = (hipStream_t)stream;
    (void)hipGetLastError();
    hipError_t e = sk::launch_rowlse(dims(shape, n), q, k, lse, st, shape->n_layers);
    if (e != hipSuccess) return device(e, "rowlse");
    return run_colsum_layers(shape, n, q, k, lse, score, accumulate, partial, st);
}

sk_status sk_recency_weight(int64_t n, double lambda, const float* in, float* out,
                            void* stream) {
    if (sk_status st = check_tokens(n)) return st;
    if (!std::isfinite(lambda) || lambda < 0.0)
        return fail(SK_E_ARG, "lambda must be finite and >= 0");
    if (n == 0) return ok();
    if (!in || !out) return fail(SK_E_ARG, "score_in and score_out must be non-NULL");
    if (!aligned(in, 4) || !aligned(out, 4))
        return fail(SK_E_ARG, "score_in and score_out must be 4-byte aligned");
    if (in != out && (const char*)in < (const char*)(out + n) &&
        (const char*)out < (const char*)(in + n))
        return fail(SK_E_ARG, "score_in and score_out overlap without being the same buffer");
    (void)hipGetLastError();
    return device(sk::launch_recency(n, lambda, in, out, (hipStream_t)stream), "recency");
}

sk_status sk_score_kvnorm(const sk_shape* shape, int64_t n, const void* k, float* score,
                          int32_t accumulate, void* stream) {
    if (sk_status st = check_shape(shape)) return st;
    if (sk_status st = check_tokens(n)) return st;
    if (accumulate != 0 && accumulate != 1) return fail(SK_E_ARG, "accumulate must be 0 or 1");
    if (n == 0) return ok();
    if (!k || !score) return fail(SK_E_ARG, "k and score must be non-NULL");
    if (!aligned(k, 16)) return fail(SK_E_ARG, "k must be 16-byte aligned");
    if (!aligned(score, 4)) return fail(SK_E_ARG, "score must be 4-byte aligned");
    (void)hipGetLastError();
    return device(sk::launch_kvnorm(dims(shape, n), k, score, accumulate, (hipStream_t)stream),
                  "kvnorm");
}

sk_status sk_balanced_keys(int64_t n, int32_t n_sink, float* keys, void* stream) {
    if (sk_status st = check_tokens(n)) return st;
    if (n_sink < 0) return fail(SK_E_ARG, "n_sink must be >= 0");
    const int64_t S = n_sink < n ? n_sink : n;
    if (n - S > ((int64_t)1 << 24))
        return fail(SK_E_UNSUPPORTED, "balanced keys are exact in fp32 for at most 2^24 tokens");
    if (n == 0) return ok();
    if (!keys) return fail(SK_E_ARG, "keys must be non-NULL");
    if (!aligned(keys, 4)) return fail(SK_E_ARG, "keys must be 4-byte aligned");
    (void)hipGetLastError();
    return device(sk::launch_balanced(n, S, keys, (hipStream_t)stream), "balanced keys");
}

size_t sk_assign_workspace_bytes(int64_t n) {
    (void)n;
    return 0;
}

sk_status sk_assign_tiers(const sk_policy* pol, const sk_plan* plan, const float* score,
                          uint32_t* map, uint32_t* order, void* ws, size_t ws_bytes,
                          void* stream) {
    (void)ws;
    (void)ws_bytes;
    if (!pol) return fail(SK_E_ARG, "policy is NULL");
    if (sk_status st = check_plan(plan, nullptr)) return st;
    if (plan->n_tokens != pol->n_tokens) return fail(SK_E_ARG, "plan and policy disagree on n_tokens");
    if (plan->n_sink != (pol->n_sink < pol->n_tokens ? pol->n_sink : pol->n_tokens))
        return fail(SK_E_ARG, "plan and policy disagree on n_sink");
    const int64_t n = plan->n_tokens;
    if (n == 0) return ok();
    if (!score || !map || !order) return fail(SK_E_ARG, "score, map and order must be non-NULL");
    if (!aligned(score, 4) || !aligned(map, 4) || !aligned(order, 4))
        return fail(SK_E_ARG, "score, map and order must be 4-byte aligned");
    (void)hipGetLastError();
    return device(sk::launch_select(n, plan->n_sink, plan->n16, plan->n8, plan->n4, score, map,
                                    order, (hipStream_t)stream),
                  "select");
}

sk_status sk_pack(const sk_shape* shape, const sk_plan* plan, const void* k, const void* v,
                  const uint32_t* map, const uint32_t* order, void* payload, void* stream) {
    (void)order;
    if (sk_status st = check_shape(shape)) return st;
    if (sk_status st = check_plan(plan, shape)) return st;
    const int64_t n = plan->n_tokens;
    if (n == 0) return ok();
    if (!k || !v || !map || !payload) return fail(SK_E_ARG, "k, v, map and payload must be non-NULL");
    if (!aligned(k, 16) || !aligned(v, 16)) return fail(SK_E_ARG, "k and v must be 16-byte aligned");
    if (!aligned(map, 4)) return fail(SK_E_ARG, "map must be 4-byte aligned");
    if (!aligned(payload, 256)) return fail(SK_E_ARG, "payload must be 256-byte aligned");
    sk::TierSeg seg[3];
    segs(plan, seg);
    (void)hipGetLastError();
    return device(sk::launch_pack(dims(shape, n), seg, k, v, map, payload, (hipStream_t)stream),
                  "pack");
}

sk_status sk_unpack(const sk_shape* shape, const sk_plan* plan, const void* payload,
                    const uint32_t* map, void* k_out, void* v_out, const sk_paged* paged,
                    void* stream) {
    if (sk_status st = check_shape(shape)) return st;
    if (sk_status st = check_plan(plan, shape)) return st;
    const int64_t n = plan->n_tokens;
    if (paged) {
        if (k_out || v_out) return fail(SK_E_ARG, "paged unpack takes k_out = v_out = NULL");
        if (paged->block_size < 1) return fail(SK_E_ARG, "block_size must be >= 1");
        if (paged->num_blocks < (n + paged->block_size - 1) / paged->block_size)
            return fail(SK_E_ARG, "num_blocks smaller than ceil(n / block_size)");
    }
    if (n == 0) return ok();
    if (!payload || !map) return fail(SK_E_ARG, "payload and map must be non-NULL");
    if (!aligned(payload, 256)) return fail(SK_E_ARG, "payload must be 256-byte aligned");
    if (!aligned(map, 4)) return fail(SK_E_ARG, "map must be 4-byte aligned");
    sk::TierSeg seg[3];
    segs(plan, seg);
    const sk::Dims d = dims(shape, n);
    (void)hipGetLastError();
    if (!paged) {
        if (!k_out || !v_out) return fail(SK_E_ARG, "dense unpack needs k_out and v_out");
        if (!aligned(k_out, 16) || !aligned(v_out, 16))
            return fail(SK_E_ARG, "k_out and v_out must be 16-byte aligned");
        return device(sk::launch_unpack_dense(d, seg, payload, map, k_out, v_out,
                                              (hipStream_t)stream),
                      "unpack");
    }
    if (!paged->k_cache || !paged->v_cache || !paged->block_table)
        return fail(SK_E_ARG, "paged unpack needs k_cache, v_cache and block_table");
    if (!aligned(paged->k_cache, 16) || !aligned(paged->v_cache, 16) ||
        !aligned(paged->block_table, 4))
        return fail(SK_E_ARG, "paged caches must be 16-byte aligned, block_table 4-byte aligned");
    return device(sk::launch_unpack_paged(d, seg, payload, map, paged->k_cache, paged->v_cache,
                                          paged->block_table, paged->block_size,
                                          paged->num_blocks, (hipStream_t)stream),
                  "unpack");
}

static size_t decode_ws(const sk_shape* shape, const sk_plan* plan, int32_t nl) {
    sk::TierSeg seg[3];
    segs(plan, seg);
    return align256((size_t)nl * (size_t)shape->n_q_heads *
                    (size_t)sk::decode_chunks(dims(shape, plan->n_tokens), seg, nl) *
                    (size_t)(shape->head_dim + 2) * sizeof(float));
}

// Decode launches put the KV head in a grid dimension, and its per-tile
// buffer ranges assume at most that many heads.
constexpr int32_t kMaxDecodeKvHeads = 65535;

size_t sk_decode_workspace_bytes(const sk_shape* shape, const sk_plan* plan, int32_t nl) {
    if (check_shape(shape) || check_plan(plan, shape) || nl < 1 || nl > shape->n_layers) return 0;
    if (shape->n_kv_heads > kMaxDecodeKvHeads) return 0;
    return decode_ws(shape, plan, nl);
}

sk_status sk_decode_attention(const sk_shape* shape, const sk_plan* plan, const void* payload,
                              int32_t layer0, int32_t nl, const void* q, float* out, float* lse,
                              void* ws, size_t ws_bytes, void* stream) {
    if (sk_status st = check_shape(shape)) return st;
    if (sk_status st = check_plan(plan, shape)) return st;
    if (nl < 1 || layer0 < 0 || (int64_t)layer0 + nl > shape->n_layers)
        return fail(SK_E_ARG, "layers [%d, %d + %d) outside [0, %d)", layer0, layer0, nl,
                    shape->n_layers);
    if (shape->n_kv_heads > kMaxDecodeKvHeads)
        return fail(SK_E_UNSUPPORTED, "decode: more than %d KV heads", kMaxDecodeKvHeads);
    if (!q || !out) return fail(SK_E_ARG, "q and out must be non-NULL");
    if (!aligned(q, 16)) return fail(SK_E_ARG, "q must be 16-byte aligned");
    if (!aligned(out, 4) || !aligned(lse, 4)) return fail(SK_E_ARG, "out and lse must be 4-byte aligned");
    const bool sent = plan->n16 + plan->n8 + plan->n4 > 0;
    if (sent && !payload) return fail(SK_E_ARG, "payload must be non-NULL");
    if (!aligned(payload, 256)) return fail(SK_E_ARG, "payload must be 256-byte aligned");
    const size_t need = decode_ws(shape, plan, nl);
    if (need && (!ws || ws_bytes < need))
        return fail(SK_E_WORKSPACE, "decode workspace needs %zu bytes, got %zu", need, ws_bytes);
    if (!aligned(ws, 16)) return fail(SK_E_ARG, "workspace must be 16-byte aligned");
    sk::TierSeg seg[3];
    segs(plan, seg);
    (void)hipGetLastError();
    return device(sk::launch_decode(dims(shape, plan->n_tokens), seg, payload, layer0, nl, q, out,
                                    lse, (float*)ws, (hipStream_t)stream),
                  "decode attention");
}

size_t sk_upgrade_bytes(const sk_shape* shape, int64_t m) {
    if (check_shape(shape) || m < 0 || m >= kMaxTokens || !kv_fits(shape, m)) return 0;
    return (size_t)shape->n_layers * (size_t)m * 2 * (size_t)shape->n_kv_heads * 2 *
           (size_t)shape->head_dim;
}

static sk_status check_upgrade(const sk_shape* shape, int64_t n, int64_t m,
                               const uint32_t* tokens, const void* payload) {
    if (sk_status st = check_shape(shape)) return st;
    if (sk_status st = check_tokens(n)) return st;
    if (m < 0 || m >= kMaxTokens) return fail(SK_E_ARG, "n_up %lld outside [0, 2^30)", (long long)m);
    if (!kv_fits(shape, n))
        return fail(SK_E_UNSUPPORTED, "shape: the fp16 KV of %lld tokens is beyond 2^62 bytes",
                    (long long)n);
    if (m == 0) return SK_OK;
    if (!tokens || !payload) return fail(SK_E_ARG, "tokens and payload must be non-NULL");
    if (!aligned(tokens, 4)) return fail(SK_E_ARG, "tokens must be 4-byte aligned");
    if (!aligned(payload, 16)) return fail(SK_E_ARG, "payload must be 16-byte aligned");
    return SK_OK;
}

sk_status sk_upgrade_pack(const sk_shape* shape, int64_t n, const void* k, const void* v,
                          const uint32_t* tokens, int64_t m, void* payload, void* stream) {
    if (sk_status st = check_upgrade(shape, n, m, tokens, payload)) return st;
    if (m == 0 || n == 0) return ok();
    if (!k || !v) return fail(SK_E_ARG, "k and v must be non-NULL");
    if (!aligned(k, 16) || !aligned(v, 16)) return fail(SK_E_ARG, "k and v must be 16-byte aligned");
    (void)hipGetLastError();
    return device(sk::launch_upgrade_pack(dims(shape, n), m, k, v, tokens, payload,
                                          (hipStream_t)stream),
                  "upgrade pack");
}

sk_status sk_upgrade_unpack(const sk_shape* shape, int64_t n, const void* payload,
                            const uint32_t* tokens, int64_t m, void* k_out, void* v_out,
                            const sk_paged* paged, void* stream) {
    if (sk_status st = check_upgrade(shape, n, m, tokens, payload)) return st;
    if (paged) {
        if (k_out || v_out) return fail(SK_E_ARG, "paged upgrade takes k_out = v_out = NULL");
        if (paged->block_size < 1) return fail(SK_E_ARG, "block_size must be >= 1");
        if (paged->num_blocks < (n + paged->block_size - 1) / paged->block_size)
            return fail(SK_E_ARG, "num_blocks smaller than ceil(n / block_size)");
    }
    if (m == 0 || n == 0) return ok();
    const sk::Dims d = dims(shape, n);
    (void)hipGetLastError();
    if (!paged) {
        if (!k_out || !v_out) return fail(SK_E_ARG, "dense upgrade needs k_out and v_out");
        if (!aligned(k_out, 16) || !aligned(v_out, 16))
            return fail(SK_E_ARG, "k_out and v_out must be 16-byte aligned");
        return device(sk::launch_upgrade_unpack(d, m, payload, tokens, k_out, v_out, nullptr, 1,
                                                0, (hipStream_t)stream),
                      "upgrade unpack");
    }
    if (!paged->k_cache || !paged->v_cache || !paged->block_table)
        return fail(SK_E_ARG, "paged upgrade needs k_cache, v_cache and block_table");
    if (!aligned(paged->k_cache, 16) || !aligned(paged->v_cache, 16) ||
        !aligned(paged->block_table, 4))
        return fail(SK_E_ARG, "paged caches must be 16-byte aligned, block_table 4-byte aligned");
    return device(sk::launch_upgrade_unpack(d, m, payload, tokens, paged->k_cache,
                                            paged->v_cache, paged->block_table,
                                            paged->block_size, paged->num_blocks,
                                            (hipStream_t)stream),
                  "upgrade unpack");
}

}  // extern "C"
