/*
 * kernel_math_check.c -- exhaustive CPU proof of the arithmetic identities
 * the gfx950 kernels use in place of slower instruction sequences.  Not part
 * of the oracle: it checks the HIP path's shortcuts against plain IEEE
 * binary32 operations (x86 SSE arithmetic and fmaf are IEEE-exact, as are
 * v_mul_f32 / v_fma_f32 / v_add_f32 with denormals enabled).
 *
 *   div   : for q in {7, 127}: with c = fl(1/q), q0 = fl(a*c),
 *           r = fma(-q0, q, a), t = fma(r, c, q0), t == fl(a/q) for every
 *           non-negative finite binary32 a (all 2^31 - 2^23 patterns).
 *   recip : for every positive finite binary16 value s and every initial
 *           estimate y0 within 2 ulp of 1/s (the hardware v_rcp_f32 is
 *           specified to 1 ulp), fma(fma(-s, y0, 1), y0, y0) == fl(1/s).
 *   magic : for every binary32 v with |v| <= 2Q, and for +-inf, NaN and
 *           every magnitude beyond (one value per exponent), with
 *           m = clamp(v, -Q, Q) (Q in {1, 7, 127}; NaN -> -Q),
 *           bits(fl(m + 1.5*2^23)) - 0x4B400000 == clamp(rint(v), -Q, Q).
 *           (Beyond 2Q the clamp maps every v of one sign to the same m.)
 *
 * Prints "OK" and exits 0 when every identity holds.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

static float bf(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t fb(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

static unsigned long long check_div(float q)
{
    const float c = 1.0f / q;
    unsigned long long bad = 0;
#pragma omp parallel for reduction(+ : bad) schedule(static)
    for (int64_t u = 0; u < 0x7F800000LL; ++u) {
        float a = bf((uint32_t)u);
        float q0 = a * c;
        float r = fmaf(-q0, q, a);
        float t = fmaf(r, c, q0);
        if (fb(t) != fb(a / q)) ++bad;
    }
    return bad;
}

static unsigned long long check_recip(void)
{
    unsigned long long bad = 0;
    for (uint32_t h = 1; h < 0x7C00u; ++h) {            /* positive finite binary16 */
        uint32_t e = (h >> 10) & 31u, f = h & 1023u;
        float s = e ? ldexpf((float)(1024u + f), (int)e - 25) : ldexpf((float)f, -24);
        float want = 1.0f / s;
        for (int d = -2; d <= 2; ++d) {
            float y0 = bf(fb(want) + (uint32_t)d);
            float err = fmaf(-s, y0, 1.0f);
            float y1 = fmaf(err, y0, y0);
            if (fb(y1) != fb(want)) ++bad;
        }
    }
    return bad;
}

static int magic_ok(float v, float Q)
{
    float m = isnan(v) ? -Q : fminf(fmaxf(v, -Q), Q);          /* v_med3_f32 */
    int32_t got = (int32_t)(fb(m + 12582912.0f) - 0x4B400000u);
    float r = rintf(v);
    float want = isnan(v) ? -Q : fminf(fmaxf(r, -Q), Q);
    return got == (int32_t)want;
}

static unsigned long long check_magic(float Q)
{
    unsigned long long bad = 0;
    const int64_t top = (int64_t)fb(2.0f * Q);
#pragma omp parallel for reduction(+ : bad) schedule(static)
    for (int64_t u = 0; u <= top; ++u) {
        if (!magic_ok(bf((uint32_t)u), Q)) ++bad;
        if (!magic_ok(bf((uint32_t)u | 0x80000000u), Q)) ++bad;
    }
    for (uint32_t e = 0; e < 256; ++e)                           /* far values, inf, NaN */
        for (uint32_t sgn = 0; sgn < 2; ++sgn)
            for (uint32_t f = 0; f < 4; ++f) {
                uint32_t u = (sgn << 31) | (e << 23) | (f * 0x1FFFFFu);
                if (!magic_ok(bf(u), Q)) ++bad;
            }
    return bad;
}

int main(void)
{
    int fail = 0;
    unsigned long long b;
    b = check_div(7.0f);   printf("div q=7     mismatches: %llu\n", b); fail |= b != 0;
    b = check_div(127.0f); printf("div q=127   mismatches: %llu\n", b); fail |= b != 0;
    b = check_recip();     printf("recip       mismatches: %llu\n", b); fail |= b != 0;
    b = check_magic(1.0f);   printf("magic Q=1   mismatches: %llu\n", b); fail |= b != 0;
    b = check_magic(7.0f);   printf("magic Q=7   mismatches: %llu\n", b); fail |= b != 0;
    b = check_magic(127.0f); printf("magic Q=127 mismatches: %llu\n", b); fail |= b != 0;
    printf(fail ? "FAIL\n" : "OK\n");
    return fail;
}
