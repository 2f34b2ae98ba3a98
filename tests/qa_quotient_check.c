/* Exhaustive check of the quotient rule the FP8 quantizers use (per row,
 * per column, and on load inside the GEMM) (page "Operator & Runtime" §5.4.3, Examples 5-7 and 5-8: the
 * code of x*448/amax).  For every bf16 amax in [2^-126, 2^118] and every
 * bf16 x with |x| <= amax (both signs, both zeros):
 *   t  = x*448                 (exact)
 *   q0 = t * RN(1/amax)
 *   e  = fma(q0, amax, -t)
 *   q1 = fma(-e, RN(1/amax), q0)
 * must have the same E4M3FN code (sign included) as RN(t/amax) clamped to
 * +-448, and |q1| must not exceed 448.  Prints "pairs <n> bad <b> over <o>". */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

static float bf16(uint32_t h)
{
    uint32_t u = h << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

/* E4M3FN code of v (|v| <= 448), round to nearest even, from the format's
 * definition: bias 7, 3 fraction bits, subnormal step 2^-9. */
static int e4m3(float v)
{
    int s = signbit(v) ? 0x80 : 0;
    float a = fabsf(v);
    if (a < 0x1p-6f) return s | (int)nearbyintf(a * 512.0f); /* 8 -> 2^-6, still right */
    int e;
    float m = frexpf(a, &e);                                   /* a = m * 2^e, m in [0.5, 1) */
    int E = e - 1, k = (int)nearbyintf((m * 2.0f - 1.0f) * 8.0f);
    if (k == 8) { k = 0; ++E; }
    return s | ((E + 7) << 3) | k;
}

int main(void)
{
    long long pairs = 0, bad = 0, over = 0;
#pragma omp parallel for schedule(dynamic, 64) reduction(+ : pairs, bad, over)
    for (int ha = 1; ha < 0x7f80; ++ha) {
        const float a = bf16((uint32_t)ha);
        if (!(a >= 0x1p-126f && a <= 0x1p118f)) continue;
        const float r = 1.0f / a;
        for (int sgn = 0; sgn < 2; ++sgn)
            for (int hx = 0; hx < 0x7f80; ++hx) {
                const float x = bf16((uint32_t)(hx | (sgn << 15)));
                if (fabsf(x) > a) break;
                const float t = x * 448.0f;
                float ref = t / a;
                if (ref > 448.0f) ref = 448.0f;
                if (ref < -448.0f) ref = -448.0f;
                const float q0 = t * r;
                const float e = fmaf(q0, a, -t);
                const float q1 = fmaf(-e, r, q0);
                ++pairs;
                if (!(fabsf(q1) <= 448.0f)) { ++over; continue; }
                if (e4m3(q1) != e4m3(ref)) ++bad;
            }
    }
    printf("pairs %lld bad %lld over %lld\n", pairs, bad, over);
    return 0;
}
