/*
 * Exhaustive check of the quotient the W4A8 activation quantiser uses in
 * place of an IEEE fp32 division a / s (kernels in w4a8.hip): with
 * r = RN(1 / s), y = RN(a * r), e = fma(-y, s, a), q = fma(e, r, y), q is the
 * correctly rounded quotient (Markstein's residual correction). The domain is
 * everything the quantiser sees: s = RN(amax / 127) for every positive finite
 * fp16 amax, and every fp16 a with |a| <= amax (every step is odd in a, so
 * a >= 0 suffices). Prints the counts and exits non-zero on any mismatch.
 * Test infrastructure, built and run by tests/test_division_identity.py.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

static float half_to_float(uint16_t h) {
    int sign = h >> 15, e = (h >> 10) & 31, m = h & 1023;
    float v = e == 0 ? ldexpf((float)m, -24) : ldexpf((float)(m | 1024), e - 25);
    return sign ? -v : v;
}

int main(void) {
    long long mismatches = 0, pairs = 0;
#pragma omp parallel for schedule(dynamic, 64) reduction(+ : mismatches, pairs)
    for (int ha = 1; ha <= 0x7BFF; ++ha) {
        const float amax = half_to_float((uint16_t)ha);
        const float s = amax / 127.0f;
        const float r = 1.0f / s;
        for (int hx = 0; hx <= ha; ++hx) {
            const float a = half_to_float((uint16_t)hx);
            const float ref = a / s;
            const float y = a * r;
            const float e = fmaf(-y, s, a);
            const float q = fmaf(e, r, y);
            uint32_t bq, br;
            memcpy(&bq, &q, 4);
            memcpy(&br, &ref, 4);
            mismatches += bq != br;
            ++pairs;
        }
    }
    printf("%lld %lld\n", pairs, mismatches);
    return mismatches != 0;
}
