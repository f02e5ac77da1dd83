// Exhaustive check of the quantize kernel's division for 16-bit weights.
//
// The kernel replaces the IEEE quotient v/S by y = 1/S (correctly rounded, once per group),
// q0 = v*y, r = fma(-q0, S, v), q1 = fma(r, y, q0), and rounds q1 to an integer.  For every
// positive finite fp16 scale S and every finite weight v (all bf16 patterns, mode 0, or all
// fp16 patterns, mode 1) with |v/S| <= 64, rint(q1) must equal rint(v/S).  Weights of a
// group satisfy |v/S| < 23 for any stored scale except the saturated 65504, for which every
// weight is checked: far quotients must stay beyond 32 with the right sign, so the code
// clamps the same way.  Built with -ffp-contract=off; fmaf is the correctly rounded fma.
// Exit status 0 when no pair disagrees.
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>
static float from_bits(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static float f16(uint32_t h) {
    uint32_t s = (h >> 15) & 1, e = (h >> 10) & 31, m = h & 1023;
    float mag;
    if (e == 0) mag = ldexpf((float)m, -24);
    else if (e == 31) mag = m ? NAN : INFINITY;
    else mag = ldexpf((float)(m | 1024), (int)e - 25);
    return s ? -mag : mag;
}
/* Mode 2: the scale's constant divisions x / 15 and x / 7 from the correctly rounded
   reciprocal and one FMA correction must equal the IEEE quotient for every finite
   non-negative fp32 x (the range x_max - x_min and max |w| are never negative). */
static int check_constant_divisions(void) {
    const float ds[2] = {15.0f, 7.0f};
    long long bad = 0;
    for (int di = 0; di < 2; ++di) {
        const float d = ds[di];
        const float c = 1.0f / d;
#pragma omp parallel for reduction(+:bad) schedule(static, 1 << 16)
        for (long long u = 0; u < 0x7F800000LL; ++u) {
            const float x = from_bits((uint32_t)u);
            const float ref = x / d;
            const float q0 = x * c;
            const float r = fmaf(-q0, d, x);
            const float q1 = fmaf(r, c, q0);
            if (memcmp(&q1, &ref, 4) != 0) ++bad;
        }
    }
    printf("constant divisions bad %lld\n", bad);
    return bad != 0;
}

int main(int argc, char** argv) {
    int mode = atoi(argv[1]);
    if (mode == 2) return check_constant_divisions();
    long long bad = 0, checked = 0, far = 0;
#pragma omp parallel for reduction(+:bad,checked,far) schedule(dynamic, 64)
    for (int sb = 1; sb < 0x7C00; ++sb) {
        const float S = f16((uint32_t)sb);
        const float y = 1.0f / S;
        for (uint32_t vb = 0; vb < 65536; ++vb) {
            const float v = mode ? f16(vb) : from_bits(vb << 16);
            if (!isfinite(v)) continue;
            const float ref = v / S;
            const float q0 = v * y;
            const float r = fmaf(-q0, S, v);
            const float q1 = fmaf(r, y, q0);
            if (fabsf(ref) <= 64.0f) {
                ++checked;
                if (rintf(q1) != rintf(ref) || fabsf(q1) > 64.0f) {
                    if (bad < 5) printf("mismatch S=%a v=%a ref=%a q1=%a\n", S, v, ref, q1);
                    ++bad;
                }
            } else if (sb == 0x7BFF) {  /* saturated scale: any weight */
                ++far;
                if (!(fabsf(q1) >= 32.0f && signbit(q1) == signbit(ref))) ++bad;
            }
        }
    }
    printf("mode %d checked %lld far %lld bad %lld\n", mode, checked, far, bad);
    return bad != 0;
}
