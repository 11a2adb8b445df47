/* Exhaustive check of the quantizer's division identity (SpectrumKV
 * Algorithm 1 "transfer": symmetric absmax codes q = rint(fl32(x / s))).
 *
 * The pack kernel does not divide per element.  With r = fl32(1 / s)
 * (one correctly rounded division per row) it computes
 *     q0 = fl32(x * r),  e = fma(-q0, s, x),  q1 = fma(e, r, q0)
 * and rounds q1.  This program checks, for every positive finite fp16 scale
 * s (normal and subnormal) and every finite fp16 x of either sign with
 * |x| <= 300 * s, that q1 is bit-identical to the correctly rounded fp32
 * quotient fl32(x / s).  300 bounds |x / s| for every row the quantizer
 * divides: x <= a = max|x|, and s = fp16_rne(fl32(a / qmax)) is at least
 * a / (2 qmax) whenever it is non-zero (qmax = 127 or 7).
 *
 * Plain C, IEEE binary32 arithmetic (build with -ffp-contract=off and
 * without -ffast-math so that every operation is rounded exactly once as
 * written; fmaf is the C library's correctly rounded fused multiply-add).
 * It also checks the two divisions that fix the row's scale (see the end of
 * main): fl32(a / qmax) by a multiply and one fused correction, and
 * fl32(1 / s) by one Newton step from any approximation within one ulp.
 * Prints "pairs=<checked> mismatches=<m> scale_checks=<c> scale_mismatches=<m>"
 * and the first mismatches; exits 1 on any mismatch (2 if its own fp16
 * decoding fails its fixed points).
 * Built with -DDROP_CORRECTION it checks q0 instead of q1, a planted mistake
 * the tests use to show that the check can fail. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

static float fp16_to_float(uint16_t h) {
    const uint32_t sign = (uint32_t)(h >> 15) << 31;
    const uint32_t exp = (h >> 10) & 0x1F;
    const uint32_t man = h & 0x3FF;
    float f;
    if (exp == 0) {
        /* zero or subnormal: man * 2^-24, exact in binary32 */
        f = ldexpf((float)man, -24);
        if (sign) f = -f;
        return f;
    }
    uint32_t bits = sign | ((exp - 15 + 127) << 23) | (man << 13);
    memcpy(&f, &bits, 4);
    return f;
}

static uint32_t bits_of(float f) {
    uint32_t b;
    memcpy(&b, &f, 4);
    return b;
}

int main(void) {
    /* positive finite fp16 values in increasing order: bit patterns 0x0001..0x7BFF */
    static float val[0x7C00];
    for (uint32_t h = 0; h < 0x7C00; ++h) val[h] = fp16_to_float((uint16_t)h);
    /* the decoder against fixed points of binary16: 2^-24, the largest
     * subnormal, 2^-14, 1, 65504, and strictly increasing values */
    if (val[1] != 0x1p-24f || val[0x3FF] != 0x3FFp-24f || val[0x400] != 0x1p-14f ||
        val[0x3C00] != 1.0f || val[0x7BFF] != 65504.0f || fp16_to_float(0xBC00) != -1.0f) {
        printf("fp16 decoding is wrong\n");
        return 2;
    }
    for (uint32_t h = 1; h < 0x7C00; ++h)
        if (!(val[h] > val[h - 1])) {
            printf("fp16 decoding is not monotonic at %u\n", h);
            return 2;
        }
    long long pairs = 0, mismatches = 0;
#pragma omp parallel for schedule(dynamic, 64) reduction(+ : pairs, mismatches)
    for (uint32_t hs = 1; hs < 0x7C00; ++hs) {
        const float s = val[hs];
        const float r = 1.0f / s;
        const float lim = 300.0f * s;
        for (uint32_t hx = 0; hx < 0x7C00 && val[hx] <= lim; ++hx) {
            for (int sg = 0; sg < 2; ++sg) {
                if (sg && hx == 0) continue;
                const float x = sg ? -val[hx] : val[hx];
                const float q0 = x * r;
#ifdef DROP_CORRECTION
                /* planted mistake (tests only): the reciprocal product alone */
                const float q1 = q0;
#else
                const float e = fmaf(-q0, s, x);
                const float q1 = fmaf(e, r, q0);
#endif
                const float ref = x / s;
                ++pairs;
                if (bits_of(q1) != bits_of(ref)) {
                    long long m;
#pragma omp atomic capture
                    m = ++mismatches;
                    if (m <= 10)
                        printf("mismatch: x=%a s=%a q1=%a x/s=%a rint %g vs %g\n", x, s, q1, ref,
                               rintf(q1), rintf(ref));
                }
            }
        }
    }
    /* The scale's two divisions, done without a divider:
     * (a) s32 = fl32(a / qmax): with rq = fl32(1 / qmax),
     *     q0 = fl32(a * rq), e = fma(-q0, qmax, a), s32 = fma(e, rq, q0),
     *     for every finite fp16 a >= 0 and qmax in {7, 127};
     * (b) r = fl32(1 / s) from any first approximation r0 within one ulp of
     *     it (the hardware reciprocal's bound): e = fma(-r0, s, 1),
     *     r = fma(e, r0, r0), for every positive finite fp16 s and each r0 in
     *     {fl32(1/s) - 1 ulp, fl32(1/s), fl32(1/s) + 1 ulp}. */
    long long scale_checks = 0, scale_mismatches = 0;
    const float qmaxes[2] = {7.0f, 127.0f};
    for (int qi = 0; qi < 2; ++qi) {
        const float qm = qmaxes[qi];
        const float rq = 1.0f / qm;
        for (uint32_t h = 0; h < 0x7C00; ++h) {
            const float a = val[h];
            const float q0 = a * rq;
#ifdef DROP_CORRECTION
            const float s32 = q0;
#else
            const float e = fmaf(-q0, qm, a);
            const float s32 = fmaf(e, rq, q0);
#endif
            ++scale_checks;
            if (bits_of(s32) != bits_of(a / qm)) {
                if (++scale_mismatches <= 5)
                    printf("scale mismatch: a=%a qmax=%g got %a want %a\n", a, qm, s32, a / qm);
            }
        }
    }
    for (uint32_t h = 1; h < 0x7C00; ++h) {
        const float s = val[h];
        const float rn = 1.0f / s;
        const float cand[3] = {nextafterf(rn, 0.0f), rn, nextafterf(rn, INFINITY)};
        for (int c = 0; c < 3; ++c) {
            const float r0 = cand[c];
#ifdef DROP_CORRECTION
            const float r = r0;
#else
            const float e = fmaf(-r0, s, 1.0f);
            const float r = fmaf(e, r0, r0);
#endif
            ++scale_checks;
            if (bits_of(r) != bits_of(rn)) {
                if (++scale_mismatches <= 5)
                    printf("reciprocal mismatch: s=%a r0=%a got %a want %a\n", s, r0, r, rn);
            }
        }
    }
    printf("pairs=%lld mismatches=%lld scale_checks=%lld scale_mismatches=%lld\n", pairs,
           mismatches, scale_checks, scale_mismatches);
    return (mismatches || scale_mismatches) ? 1 : 0;
}
