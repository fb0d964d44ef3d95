/* CPU check of the division step used by the E4M3 V store for scales d in
 * [2^-64, 2^64]: q0 = RN(x r) with r = RN(1/d) (from a double division),
 * q1 = RN(q0 + RN?(x - q0 d) r) by two fused multiply-adds, sign of q0 kept,
 * no correction for |q0| >= 1e30.  Reads "d count seed" lines; for each d
 * draws `count` x = RN(q d) with |q| log-uniform in [2^-12, 2^10] (the
 * quotients whose E4M3 code depends on their rounding) and random sign, plus
 * the x whose quotients sit next to every E4M3 rounding midpoint, and prints
 * the number of x whose q1 differs from the IEEE quotient x / d. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

static uint64_t st;
static uint64_t next(void)
{
    st ^= st << 13; st ^= st >> 7; st ^= st << 17;
    return st;
}

static float step(float x, float d, float r)
{
    float q0 = x * r;
    float q1 = fmaf(fmaf(-q0, d, x), r, q0);
    return copysignf(fabsf(q0) < 1e30f ? q1 : q0, q0);
}

static int differs(float x, float d, float r)
{
    float a = x / d, b = step(x, d, r);
    uint32_t ua, ub;
    memcpy(&ua, &a, 4);
    memcpy(&ub, &b, 4);
    return ua != ub;
}

int main(void)
{
    double dd;
    long count;
    unsigned long long seed;
    while (scanf("%lf %ld %llu", &dd, &count, &seed) == 3) {
        float d = (float)dd, r = (float)(1.0 / (double)d);
        st = seed | 1;
        long bad = 0, n = 0;
        for (long i = 0; i < count; ++i, ++n) {
            double u = (double)(next() >> 11) / 9007199254740992.0;
            double q = ldexp(1.0, -12) * pow(2.0, 22.0 * u);
            float x = (float)(q * (double)d);
            if (next() & 1) x = -x;
            bad += differs(x, d, r);
        }
        /* E4M3 rounding midpoints m (between neighbouring E4M3 values up to
         * 448: (k + 1/2) 2^-9 in the subnormal range, (1 + (k + 1/2) / 8) 2^e
         * above): the floats x nearest m d, and 64 floats on either side */
        for (int e = -7; e <= 8; ++e)
            for (int k = 0; k < 8; ++k) {
                double m = e < -6 ? (k + 0.5) * ldexp(1.0, -9) : ldexp(1.0 + (k + 0.5) / 8.0, e);
                float x = (float)(m * (double)d);
                uint32_t b;
                memcpy(&b, &x, 4);
                for (int j = -64; j <= 64; ++j, ++n) {
                    uint32_t bj = b + (uint32_t)j;
                    float xj;
                    memcpy(&xj, &bj, 4);
                    bad += differs(xj, d, r) + differs(-xj, d, r);
                    ++n;
                }
            }
        printf("%.9g %ld %ld\n", (double)d, n, bad);
    }
    return 0;
}
