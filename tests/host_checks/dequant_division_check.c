/* Host check of the division the dequantization kernel uses instead of IEEE
 * division by the FP32 tensor scale.
 *
 *  t   = fl(r * s)       r: decoded element of any block format on E4M3 scales: an
 *                         E2M1 value (NVFP4, IF4, Four Over Six), an FP3 E2M0 value
 *                         (IF3), an FP6 E2M3 value (IF6), or an INT restore: q (NVINT4,
 *                         q in -8..7), fl(q * fl(6/7)) (IF4), fl(q * fl(4/3)) (IF3, q in
 *                         -4..3), fl(q * fl(7.5/31)) (IF6, q in -32..31);
 *                         s: decoded E4M3 block scale
 *  out = fl(t / gs)      wanted, correctly rounded
 *  div_rs(t, gs, rg) = fma(-fma(q0, gs, -t), rg, q0),  q0 = fl(t * rg),  rg = fl(1 / gs)
 *
 * The kernel takes div_rs only when ratio = fl(s * rg) lies in [2^-98, 2^96], and
 * IEEE division otherwise. Claims checked (exit status 0 only if all hold):
 *  1. Over all element codes and all E4M3 scale codes, the nonzero dividends t have
 *     few distinct significands; div_rs is correctly rounded for each of them against
 *     every one of the 2^23 divisor significands, in both quotient binades.
 *  2. Random spot checks across the exponent range the ratio predicate admits
 *     (real codes, random gs), both signs, reproduce IEEE division bit for bit.
 *  3. Zero dividends of either sign keep their sign.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

static float div_rs(float t, float s, float rs)
{
    float q0 = t * rs;
    float res = -fmaf(q0, s, -t);
    return fmaf(res, rs, q0);
}

static float e4m3(int code)
{
    int e = (code >> 3) & 15, m = code & 7;
    return e == 0 ? ldexpf((float)m, -9) : ldexpf((float)(8 + m), e - 10);
}

/* element value of code `c` in format `fmt`:
 *   0 E2M1, 1 INT4 times fl(6/7), 2 INT4 (NVINT4), 3 FP3 E2M0, 4 INT3 times fl(4/3),
 *   5 FP6 E2M3, 6 INT6 times fl(7.5/31) */
#define NFMT 7
static const int fmt_codes[NFMT] = {16, 16, 16, 8, 8, 64, 64};
static float element(int fmt, int c)
{
    static const float mag[8] = {0.0f, 0.5f, 1.0f, 1.5f, 2.0f, 3.0f, 4.0f, 6.0f};
    switch (fmt) {
    case 0: return (c & 8) ? -mag[c & 7] : mag[c & 7];
    case 1: return (float)(((c ^ 8) - 8)) * (6.0f / 7.0f);
    case 2: return (float)((c ^ 8) - 8);
    case 3: { float m = (c & 3) ? ldexpf(1.0f, (c & 3) - 1) : 0.0f; return (c & 4) ? -m : m; }
    case 4: return (float)(((c ^ 4) - 4)) * (4.0f / 3.0f);
    case 5: { int e = (c >> 3) & 3, m = c & 7;     /* E2M3: bias 1, subnormals at e = 0 */
              float v = e ? ldexpf(1.0f + m / 8.0f, e - 1) : m / 8.0f;
              return (c & 32) ? -v : v; }
    default: return (float)(((c ^ 32) - 32)) * (7.5f / 31.0f);
    }
}

static int same(float a, float b) { return memcmp(&a, &b, 4) == 0; }

/* argv[1], optional: check every n-th divisor significand only (the sanitizer build,
 * which looks for memory errors and undefined behaviour, not for coverage). */
int main(int argc, char** argv)
{
    const uint32_t stride = argc > 1 ? (uint32_t)atoi(argv[1]) : 1u;
    static float sig[4096];
    int nsig = 0;
    for (int fmt = 0; fmt < NFMT; ++fmt)
        for (int nib = 0; nib < fmt_codes[fmt]; ++nib)
            for (int code = 1; code <= 0x7E; ++code) {
                float t = fabsf(element(fmt, nib) * e4m3(code));
                if (t == 0.0f) continue;
                int e;
                float m = 2.0f * frexpf(t, &e); /* [1, 2) */
                int dup = 0;
                for (int k = 0; k < nsig && !dup; ++k) dup = sig[k] == m;
                if (!dup) sig[nsig++] = m;
            }

    long checked = 0, bad = 0;
    for (uint32_t mant = 0; mant < (1u << 23); mant += (stride ? stride : 1u)) {
        uint32_t bits = 0x3F800000u | mant;
        float y;
        memcpy(&y, &bits, 4);
        float ry = 1.0f / y;
        for (int k = 0; k < nsig; ++k) {
            float t = sig[k], t2 = 2.0f * sig[k];
            if (!same(div_rs(t, y, ry), t / y)) ++bad;
            if (!same(div_rs(t2, y, ry), t2 / y)) ++bad;
            checked += 2;
        }
    }

    /* 2: spot checks over the admitted exponent range */
    long spot = 0, spot_bad = 0;
    uint32_t lcg = 2463534242u;
    for (int k = 0; k < 6000000; ++k) {
        lcg = lcg * 1664525u + 1013904223u;
        uint32_t mant = lcg >> 9;
        lcg = lcg * 1664525u + 1013904223u;
        int ex = (int)(lcg % 230u) - 115;
        int code = 1 + (int)((lcg >> 8) % 126u);
        int fmt = (int)((lcg >> 20) % NFMT), nib = (int)((lcg >> 12) % (uint32_t)fmt_codes[fmt]);
        uint32_t bits = 0x3F800000u | mant;
        float gs;
        memcpy(&gs, &bits, 4);
        gs = ldexpf(gs, ex);
        if (lcg & 0x80000000u) gs = -gs; /* negative scales must take the slow path */
        float s = e4m3(code), rg = 1.0f / gs, ratio = s * rg;
        if (!(ratio >= 0x1p-98f && ratio <= 0x1p+96f)) continue;
        float t = element(fmt, nib) * s;
        if (!same(div_rs(t, gs, rg), t / gs)) ++spot_bad;
        ++spot;
    }

    /* 3: signed zeros */
    int zero_bad = 0;
    for (int code = 1; code <= 0x7E; ++code) {
        float gs = e4m3(code) * 3.7f, rg = 1.0f / gs;
        float a = div_rs(-0.0f, gs, rg), b = div_rs(0.0f, gs, rg);
        if (!(a == 0.0f && signbit(a) && b == 0.0f && !signbit(b))) ++zero_bad;
    }

    printf("%d dividend significands; exhaustive checked %ld, mismatches %ld; spot checked %ld, "
           "mismatches %ld; signed-zero failures %d\n", nsig, checked, bad, spot, spot_bad, zero_bad);
    return (bad == 0 && spot_bad == 0 && zero_bad == 0 && spot > 1000000) ? 0 : 1;
}
