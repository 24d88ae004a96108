/* Host check of the arithmetic the HIP kernels use in place of IEEE division by a
 * block scale.
 *
 *  recip(s, r0) = fma(fma(-s, r0, 1), r0, r0)      r0: hardware estimate of 1/s
 *  pair(s):  zh = recip(s) stepped one ulp down if s*zh > 1,
 *            zl = fl(fma(-s, zh, 1) * zh)
 *  div2(t)   = fma(t, zh, t*zl)
 *
 * Claims checked (exit status 0 only if all hold):
 *  1. recip returns fl(1/s) for all 126 positive E4M3 values and 6, for any r0
 *     among fl(1/s) and its two neighbours.
 *  2. div2 equals the correctly rounded t/s for every binary32 significand of t and
 *     each of the eight divisor significands 1, 1.125, ..., 1.875 (this covers every
 *     E4M3 value and 6 up to a power of two); exponents are spot-checked with the
 *     actual E4M3 divisors for |t| in [2^-90, 2^90), both signs.
 *  3. div2 keeps the sign of a zero dividend, and the zero pair maps every t to a
 *     zero of t's sign.
 *  4. The constants the kernels use for dividing by 6 are pair(6).
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

static float recip(float s, float r0) { return fmaf(fmaf(-s, r0, 1.0f), r0, r0); }

typedef struct { float zh, zl; } pair_t;

static pair_t make_pair(float s, float r0)
{
    pair_t p;
    float zh = recip(s, r0);
    float e = fmaf(-s, zh, 1.0f);
    if (e < 0.0f) {
        uint32_t b;
        memcpy(&b, &zh, 4);
        b -= 1u;
        memcpy(&zh, &b, 4);
        e = fmaf(-s, zh, 1.0f);
    }
    p.zh = zh;
    p.zl = e * zh;
    return p;
}

static float div2(float t, pair_t p) { return fmaf(t, p.zh, t * p.zl); }

static float e4m3(int code)
{
    int e = (code >> 3) & 15, m = code & 7;
    return e == 0 ? ldexpf((float)m, -9) : ldexpf((float)(8 + m), e - 10);
}

static int same(float a, float b) { return memcmp(&a, &b, 4) == 0; }

int main(void)
{
    long bad_rcp = 0, bad_div = 0, checked = 0, bad_zero = 0;

    /* 1: reciprocal, from any estimate within one ulp */
    for (int code = 1; code <= 0x7F; ++code) {
        float s = code == 0x7F ? 6.0f : e4m3(code), ref = 1.0f / s;
        float cands[3] = {ref, nextafterf(ref, INFINITY), nextafterf(ref, 0.0f)};
        pair_t p0 = make_pair(s, ref);
        for (int c = 0; c < 3; ++c) {
            if (!same(recip(s, cands[c]), ref)) ++bad_rcp;
            pair_t p = make_pair(s, cands[c]);
            if (!same(p.zh, p0.zh) || !same(p.zl, p0.zl)) ++bad_rcp;
        }
    }

    /* 2: every dividend significand against every divisor significand */
    for (int m = 8; m < 16; ++m) {
        float s = (float)m / 8.0f;
        pair_t p = make_pair(s, 1.0f / s);
        for (uint32_t mant = 0; mant < (1u << 23); ++mant) {
            uint32_t bits = 0x3F800000u | mant;
            float t;
            memcpy(&t, &bits, 4);
            if (!same(div2(t, p), t / s)) ++bad_div;
            ++checked;
        }
    }
    /* exponent spot checks with the actual divisors */
    uint32_t lcg = 12345u;
    for (int k = 0; k < 4000000; ++k) {
        lcg = lcg * 1664525u + 1013904223u;
        uint32_t mant = lcg >> 9;
        lcg = lcg * 1664525u + 1013904223u;
        int ex = (int)(lcg % 180u) - 90;                /* |t| in [2^-90, 2^90) */
        int code = 1 + (int)((lcg >> 8) % 126u);
        uint32_t bits = 0x3F800000u | mant;
        float t;
        memcpy(&t, &bits, 4);
        t = ldexpf(t, ex);
        if (lcg & 1u) t = -t;
        float s = e4m3(code);
        if (!same(div2(t, make_pair(s, 1.0f / s)), t / s)) ++bad_div;
        ++checked;
    }

    /* 3: signed zeros */
    pair_t zero = {0.0f, 0.0f};
    for (int code = 1; code <= 0x7E; ++code) {
        float s = e4m3(code);
        pair_t p = make_pair(s, 1.0f / s);
        float nz = div2(-0.0f, p), pz = div2(0.0f, p);
        if (!(signbit(nz) && !signbit(pz) && nz == 0.0f && pz == 0.0f)) ++bad_zero;
    }
    {
        float a = div2(-1.5f, zero), b = div2(3.0f, zero);
        if (!(a == 0.0f && signbit(a) && b == 0.0f && !signbit(b))) ++bad_zero;
    }

    /* 4: the division-by-6 constants */
    pair_t p6 = make_pair(6.0f, 1.0f / 6.0f);
    uint32_t zh6, zl6;
    memcpy(&zh6, &p6.zh, 4);
    memcpy(&zl6, &p6.zl, 4);
    int six_ok = zh6 == 0x3E2AAAAAu && zl6 == 0x322AAAAAu;

    printf("recip/pair mismatches %ld; div2 checked %ld, mismatches %ld; signed-zero failures %ld; "
           "six pair %08x %08x %s\n", bad_rcp, checked, bad_div, bad_zero, zh6, zl6, six_ok ? "ok" : "WRONG");
    return (bad_rcp == 0 && bad_div == 0 && bad_zero == 0 && six_ok) ? 0 : 1;
}
