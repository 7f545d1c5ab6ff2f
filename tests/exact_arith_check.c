/* Exhaustive checks of two float32 sequences the page writers use instead of IEEE division:
 *  1. x / d for d in {3, 15, 255}: q0 = RN(x * RN(1/d)), r = fma(-q0, d, x), q = fma(r, RN(1/d), q0)
 *     equals the correctly rounded x / d for every positive finite float x.  Every x below
 *     2^-87 (biased exponent <= 40: all cases where q0, r or q can be subnormal) is tried;
 *     above, q0, r and q are normal or zero and scale exactly with x's power of two, so one
 *     binade's 2^23 mantissas decide every binade; five whole binades up to the largest are
 *     tried;
 *  2. 1 / y for y a positive finite fp16 value: r = fma(fma(-y, r0, 1), r0, r0) equals the
 *     correctly rounded 1 / y for every seed r0 within 2 ulp of it.
 * Prints the number of mismatches of each check; exit status 0 when both are zero. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

static float f_of(uint32_t u) { float x; memcpy(&x, &u, 4); return x; }
static uint32_t u_of(float x) { uint32_t r; memcpy(&r, &x, 4); return r; }

static float half_value(uint32_t h) {
    const int e = (int)((h >> 10) & 31u), m = (int)(h & 1023u);
    return e == 0 ? ldexpf((float)m, -24) : ldexpf((float)(m | 1024), e - 25);
}

int main(void) {
    const float ds[3] = {3.0f, 15.0f, 255.0f};
    long long bad_div = 0;
    for (int k = 0; k < 3; ++k) {
        const float d = ds[k];
        const float c = 1.0f / d;
        long long bad = 0;
        const long long binades[5] = {41, 100, 127, 200, 254};
        const long long n_low = 41LL << 23, n = n_low + 5 * (1LL << 23);
#pragma omp parallel for reduction(+ : bad) schedule(static)
        for (long long i = 0; i < n; ++i) {
            const long long b = i < n_low ? i : (binades[(i - n_low) >> 23] << 23) | ((i - n_low) & 0x7fffff);
            const float x = f_of((uint32_t)b);
            const float q0 = x * c;
            const float r = fmaf(-q0, d, x);
            const float q = fmaf(r, c, q0);
            if (u_of(q) != u_of(x / d)) ++bad;
        }
        printf("division by %g: %lld mismatches\n", d, bad);
        bad_div += bad;
    }
    long long bad_rcp = 0;
    for (uint32_t h = 1; h < 0x7c00u; ++h) {
        const float y = half_value(h);
        const float ref = 1.0f / y;
        for (int delta = -2; delta <= 2; ++delta) {
            const float r0 = f_of(u_of(ref) + (uint32_t)delta);
            const float r = fmaf(fmaf(-y, r0, 1.0f), r0, r0);
            if (u_of(r) != u_of(ref)) ++bad_rcp;
        }
    }
    printf("fp16 reciprocal: %lld mismatches\n", bad_rcp);
    return (bad_div == 0 && bad_rcp == 0) ? 0 : 1;
}
