/* Host check of the per-token activation quantizer's division-free rounding.
 *
 * The kernel (actquant.hip) computes q = rint(x / s) for fp16 x and the fp16
 * row scale s = fp16(max|x| / 127) without a division per element:
 *     f  = x * RN(1/s)
 *     qf = floor(f) + 1/2
 *     q  = rint(fma(qf, s, -x) == 0 ? qf : f)
 * and, to save most of that work, first tries q = rint(f) and keeps it unless
 * f lies within NEAR_MARGIN (2^-15) of a half-integer (|f - x/s| <= 127 * 2^-23,
 * about 1.5e-5, so only such f can round differently from x / s), in which case
 * the steps above decide.
 * This program replays those fp32 steps and compares them with rint(x / s)
 * (IEEE fp32 division, itself bit-exact with the real quotient for fp16
 * operands) for every positive finite fp16 row maximum a and every fp16 x
 * with |x| <= a.  Exit status 0 means no pair differs.  Build with
 * -ffp-contract=off so the compiler adds no fusion of its own. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

static float h2f(uint16_t h) {
    const uint32_t sgn = (h >> 15) & 1, e = (h >> 10) & 31, m = h & 1023;
    const float v = e == 0 ? ldexpf((float)m, -24) : ldexpf((float)(m | 1024), (int)e - 25);
    return sgn ? -v : v;
}

/* fp32 -> fp16 bits, round to nearest even (finite, |f| < 65520) */
static uint16_t f2h(float f) {
    uint32_t x;
    memcpy(&x, &f, 4);
    const uint32_t sign = (x >> 16) & 0x8000u, ax = x & 0x7FFFFFFFu;
    if (ax < 0x38800000u) { /* below 2^-14: a subnormal half, in units of 2^-24 */
        float af;
        memcpy(&af, &ax, 4);
        return (uint16_t)(sign | (uint32_t)rintf(af * 16777216.0f));
    }
    uint32_t h = (((ax >> 23) - 112u) << 10) | ((ax & 0x7FFFFFu) >> 13);
    const uint32_t rem = ax & 0x1FFFu;
    if (rem > 0x1000u || (rem == 0x1000u && (h & 1u))) h++;
    return (uint16_t)(sign | h);
}

#ifndef NEAR_MARGIN
#define NEAR_MARGIN 0x1p-15f
#endif

int main(void) {
    long long bad = 0, total = 0, ties = 0, near_count = 0;
#pragma omp parallel for reduction(+ : bad, total, ties, near_count) schedule(dynamic, 64)
    for (int ah = 1; ah < 0x7C00; ah++) {
        const float a = h2f((uint16_t)ah);
        const float s = h2f(f2h(a / 127.0f));
        const float sd = s == 0.0f ? 1.0f : s;
        const float r = 1.0f / sd;
        for (int xh = 0; xh <= ah; xh++)
            for (int neg = 0; neg < 2; neg++) {
                const float x = neg ? -h2f((uint16_t)xh) : h2f((uint16_t)xh);
                const float ref = rintf(x / sd);
                const float f = x * r;
                const float qf = floorf(f) + 0.5f;
                const float t = fmaf(qf, sd, -x);
#ifdef DROP_TIE_TEST /* the mutant the test suite expects to fail */
                const float qe = rintf(f);
#else
                const float qe = rintf(t == 0.0f ? qf : f);
#endif
                /* the kernel's fast path: rint(f) unless f is near a half-integer */
                const float q0 = rintf(f);
                const int near = fabsf(f - q0) >= 0.5f - NEAR_MARGIN;
                const float q = near ? qe : q0;
                total++;
                ties += t == 0.0f;
                near_count += near;
                bad += q != ref;
            }
    }
    printf("pairs %lld exact ties %lld near half-integers %lld mismatches %lld\n", total, ties, near_count, bad);
    return bad != 0;
}
