/* Exhaustive check of the quotient rule of the fixed-range E4M3FN output of
 * SwiGLU (page "Operator & Runtime" §5.3.1: Z stored with one fixed scale
 * factor; the code of z*448/amax).  z = t*u is a product of two bf16
 * values, so its significand has at most 16 bits; amax is a bf16 value;
 * |z| <= amax (larger |z| saturate before the quotient).
 * For every such pair
 *   t  = z*448                 (exact: at most 19 significant bits)
 *   q0 = t * RN(1/amax)
 *   e  = fma(q0, amax, -t)
 *   q1 = fma(-e, RN(1/amax), q0)
 * must give the same E4M3FN code (sign included) as RN(t/amax), and |q1|
 * must not exceed 448, for amax in [2^-80, 2^118] (below that the residual
 * e of small quotients is subnormal and the rule fails: at amax near
 * 2^-126 some codes differ by one).
 *
 * Every operation here is invariant under scaling z and amax by one power
 * of two while every intermediate stays a normal number, which holds for
 * amax in [2^-80, 2^118] and z within 2^30 of amax (t, the residual, q0
 * and q1 are then normal).  So the check takes amax's 128 significands in
 * the binade [1, 2) with every 16-bit significand of z and every binade of
 * z from amax's down to 30 below it (quotients under 2^-11 give code 0;
 * smaller z give quotients below 2^-20, where q1, like RN(t/amax), is a
 * tiny or zero value of z's sign: code 0 with that sign),
 * and, for the two ends, the binades 2^-80 and 2^117 and amax = 2^118 with
 * z down to 24 binades below; both signs.  Prints "pairs <n> bad <b> over
 * <o>". */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

/* E4M3FN code of v (|v| <= 448), round to nearest even, from the format's
 * definition: bias 7, 3 fraction bits, subnormal step 2^-9. */
static int e4m3(float v)
{
    int s = signbit(v) ? 0x80 : 0;
    float a = fabsf(v);
    if (a < 0x1p-6f) return s | (int)nearbyintf(a * 512.0f);
    int e;
    float m = frexpf(a, &e);
    int E = e - 1, k = (int)nearbyintf((m * 2.0f - 1.0f) * 8.0f);
    if (k == 8) { k = 0; ++E; }
    return s | ((E + 7) << 3) | k;
}

static long long check(float a, int shifts, long long *bad, long long *over)
{
    const float r = 1.0f / a;
    long long pairs = 0;
    int ea;
    (void)frexpf(a, &ea);
    for (int shift = 0; shift <= shifts; ++shift)
        for (int mz = 0; mz < (1 << 15); ++mz)
            for (int sgn = 0; sgn < 2; ++sgn) {
                /* z = (1 + mz/2^15) 2^(ea - 1 - shift): 16 significant bits */
                float z = ldexpf(1.0f + (float)mz / 32768.0f, ea - 1 - shift);
                if (sgn) z = -z;
                if (fabsf(z) > a) continue;
                const float t = z * 448.0f;
                const float ref = t / a;
                const float q0 = t * r;
                const float e = fmaf(q0, a, -t);
                const float q1 = fmaf(-e, r, q0);
                ++pairs;
                if (!(fabsf(q1) <= 448.0f)) { ++*over; continue; }
                if (e4m3(q1) != e4m3(ref)) ++*bad;
            }
    return pairs;
}

int main(void)
{
    long long pairs = 0, bad = 0, over = 0;
    static const int binades[3] = {0, -80, 117};
    static const int shifts[3] = {30, 24, 24};
#pragma omp parallel for schedule(dynamic, 1) collapse(2) reduction(+ : pairs, bad, over)
    for (int b = 0; b < 3; ++b)
        for (int ma = 0; ma < 128; ++ma) {
            const float a = ldexpf(1.0f + (float)ma / 128.0f, binades[b]);
            pairs += check(a, shifts[b], &bad, &over);
        }
    pairs += check(0x1p118f, 24, &bad, &over);
    printf("pairs %lld bad %lld over %lld\n", pairs, bad, over);
    return 0;
}
