/*
 * fp4q_oracle.c -- CPU oracle for block-scaled FP4 quantization.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may call this file:
 * only tests/, the smoke check and the benchmark's CPU-baseline leg load it.
 * It shares no code, header, table or constant generator with the HIP library.
 *
 * Plain, slow, single-threaded C99.  Every floating-point operation is an IEEE
 * binary32 operation rounded to nearest-even unless stated otherwise; build with
 * -O1 -ffp-contract=off and never with -ffast-math, so that fl(a*b) and fl(a+b)
 * stay separate roundings.  fmaf() is used only where the reading adopted below
 * asks for one fused rounding.
 *
 * Sources (cited by page and section, nothing else):
 *  [NV]  qiita.com/nishiha/items/b98c2b931d588c4c81d5 -- notes on NVIDIA's NVFP4
 *        pretraining recipe; sections "NVFP4フロー図" (the three GEMMs on quantized
 *        operands), "NVFP4データの変換" (E2M1), "2D scaling",
 *        "ランダムアダマール変換" (RHT), "確率的丸め" (SR), "NVFP4の表現できる最大値",
 *        "scaleの導出" (two-level scale).
 *  [GL]  ultralytics.com/ja/glossary/fp4 -- glossary "FP4"; section "FP4の仕組み"
 *        (MXFP4 / NVFP4 definitions and the block-size MAE snippet), section
 *        "FP4による推論と学習" (FP4 products accumulated in higher precision).
 *  [IF]  gist.science/ja/paper/2603.28765 -- explainer of "Adaptive Block-Scaled
 *        Data Types"; section "2. 提案手法：IF4" (IF4, the sign-bit flag, the 6/7
 *        rule) and section "3. 主要な貢献" (Table 1).
 *  [F6]  blog.ast.moe/blog/2026-09-24 -- "FP6から考えるLLM量子化"; section
 *        "FP6で隣り合う値の間隔を見てみる" (E8M0 conversion with round-to-nearest-even).
 *  [PX]  Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers: As Easy as 1, 2, 3",
 *        SC'11 -- the Philox4x32-10 counter-based generator (not on the pages; the
 *        method asks for a Philox stream keyed on (seed, element index)).
 *
 * Readings taken where the pages are silent are listed in the repository's design
 * notes; each function states the one it uses.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>
#include <float.h>

#include "fp4q_oracle.h"

/* ------------------------------------------------------------------------- */
/* Philox4x32-10 [PX]                                                         */
/* ------------------------------------------------------------------------- */

/* Ten rounds of the Philox-4x32 bijection.  One round multiplies counter words 0
 * and 2 by the two round constants (full 64-bit products), then permutes and
 * whitens with the round key: new = (hi(M1*c2)^c1^k0, lo(M1*c2), hi(M0*c0)^c3^k1,
 * lo(M0*c0)).  The key is advanced by the two Weyl constants between rounds. */
void ora_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4])
{
    const uint32_t M0 = 0xD2511F53u, M1 = 0xCD9E8D57u;
    const uint32_t W0 = 0x9E3779B9u, W1 = 0xBB67AE85u;
    uint32_t c0 = ctr[0], c1 = ctr[1], c2 = ctr[2], c3 = ctr[3];
    uint32_t k0 = key[0], k1 = key[1];
    for (int round = 0; round < 10; ++round) {
        if (round > 0) {
            k0 += W0;
            k1 += W1;
        }
        uint64_t p0 = (uint64_t)M0 * (uint64_t)c0;
        uint64_t p1 = (uint64_t)M1 * (uint64_t)c2;
        uint32_t n0 = (uint32_t)(p1 >> 32) ^ c1 ^ k0;
        uint32_t n1 = (uint32_t)p1;
        uint32_t n2 = (uint32_t)(p0 >> 32) ^ c3 ^ k1;
        uint32_t n3 = (uint32_t)p0;
        c0 = n0; c1 = n1; c2 = n2; c3 = n3;
    }
    out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

/* The 16-bit uniform used by stochastic rounding for element `idx` (row-major index
 * in the logical quantized matrix) of stream `stream` (0: row-wise, 2D and MXFP4
 * outputs; 1: the column-wise output, i.e. the matrix X^T).  One Philox call serves
 * eight consecutive elements: counter {lo32(idx/8), hi32(idx/8), stream, 0}, key
 * {lo32(seed), hi32(seed)}; element idx takes a 16-bit half of word (idx / 2) & 3,
 * the high half for even idx and the low half for odd idx. */
uint32_t ora_sr_bits16(uint64_t seed, uint32_t stream, uint64_t idx)
{
    uint64_t group = idx >> 3;
    uint32_t ctr[4] = {(uint32_t)group, (uint32_t)(group >> 32), stream, 0u};
    uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
    uint32_t out[4];
    ora_philox4x32_10(ctr, key, out);
    uint32_t word = out[(idx >> 1) & 3];
    return (idx & 1) ? (word & 0xFFFFu) : (word >> 16);
}

/* The RHT's random diagonal S: 128 signs from one Philox call with counter
 * {0,0,0,1} (the last word keeps this stream apart from the SR stream) and key
 * {lo32(seed), hi32(seed)}.  Bit t (word t/32, bit t%32) set means s_t = -1. */
void ora_rht_signs(uint64_t seed, uint32_t signs[4])
{
    uint32_t ctr[4] = {0u, 0u, 0u, 1u};
    uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
    ora_philox4x32_10(ctr, key, signs);
}

/* ------------------------------------------------------------------------- */
/* E2M1 element format [NV "NVFP4データの変換"], [GL "FP4の仕組み"]               */
/* ------------------------------------------------------------------------- */

/* Magnitudes of the eight non-negative E2M1 codes: e=0 gives 0.5*m, e>0 gives
 * (1 + 0.5*m) * 2^(e-1), for the 3-bit magnitude code (e1 e0 m). */
static const float E2M1_MAG[8] = {0.0f, 0.5f, 1.0f, 1.5f, 2.0f, 3.0f, 4.0f, 6.0f};

/* Nibble layout s e1 e0 m: bit 3 is the sign. */
float ora_e2m1_decode(uint8_t nibble)
{
    float m = E2M1_MAG[nibble & 7];
    return (nibble & 8) ? -m : m;
}

/* Round-to-nearest onto the E2M1 grid.  Reading: ties go to the even code (the
 * IEEE default; the code's last bit is the mantissa bit), magnitudes beyond 6
 * saturate to 6 (E2M1 has no infinity), and the sign bit is copied from v so -0
 * and small negatives give 0x8. */
uint8_t ora_e2m1_rtn(float v)
{
    double a = fabs((double)v);
    if (a >= 6.0) return (uint8_t)(7 | (signbit(v) ? 8 : 0));   /* at or beyond the maximum */
    int best = 0;
    double best_d = a;                     /* distance to magnitude 0 */
    for (int c = 1; c < 8; ++c) {
        double d = fabs(a - (double)E2M1_MAG[c]);
        if (d < best_d || (d == best_d && (c & 1) == 0)) {
            best = c;
            best_d = d;
        }
    }
    return (uint8_t)(best | (signbit(v) ? 8 : 0));
}

/* Stochastic rounding onto the E2M1 grid [NV "確率的丸め"]: the page's
 * Round(x + U(-1/2, 1/2)) on a unit grid is floor(x + u) with u ~ U[0, 1).  On the
 * E2M1 grid this is done on the local interval [lo, hi] that holds a = |v|:
 * with frac = (a - lo) / (hi - lo) the value rounds up iff frac + u >= 1, where
 * u = r16 / 2^16 comes from the Philox stream.  |v| >= 6 gives 6.  Sign copied. */
uint8_t ora_e2m1_sr(float v, uint32_t r16)
{
    double a = fabs((double)v);
    int c;
    if (a >= 6.0) {
        c = 7;
    } else {
        int lo = 0;
        for (int k = 0; k < 7; ++k)
            if ((double)E2M1_MAG[k] <= a) lo = k;
        double step = (double)E2M1_MAG[lo + 1] - (double)E2M1_MAG[lo];
        double frac = (a - (double)E2M1_MAG[lo]) / step;      /* exact in binary64 */
        double u = (double)(r16 & 0xFFFFu) / 65536.0;
        c = (frac >= 1.0 - u) ? lo + 1 : lo;                   /* frac + u >= 1, exactly */
    }
    return (uint8_t)(c | (signbit(v) ? 8 : 0));
}

/* ------------------------------------------------------------------------- */
/* E4M3 (fn) block scale [NV "NVFP4の表現できる最大値", "scaleの導出"]            */
/* ------------------------------------------------------------------------- */

/* Value of a non-negative E4M3 code: exponent bias 7, subnormal step 2^-9. */
float ora_e4m3_decode(uint8_t code)
{
    int e = (code >> 3) & 15, m = code & 7;
    double v = (e == 0) ? ldexp((double)m, -9) : ldexp((double)(8 + m), e - 10);
    return (float)((code & 0x80) ? -v : v);
}

/* Nearest non-negative E4M3 value to y >= 0 by exhaustive search over the 127
 * finite codes 0x00..0x7E; ties go to the even code.  y >= 448 (the format's
 * maximum) saturates to 0x7E; 0x7F (NaN) is never produced. */
uint8_t ora_e4m3_encode(float y)
{
    if (!(y > 0.0f)) return 0;
    if (y >= 448.0f) return 0x7E;
    int best = 0;
    double best_d = (double)y;
    for (int c = 1; c <= 0x7E; ++c) {
        double d = fabs((double)y - (double)ora_e4m3_decode((uint8_t)c));
        if (d < best_d || (d == best_d && (c & 1) == 0)) {
            best = c;
            best_d = d;
        }
    }
    return (uint8_t)best;
}

/* ------------------------------------------------------------------------- */
/* E8M0 power-of-two scale [GL "FP4の仕組み"], [F6]                              */
/* ------------------------------------------------------------------------- */

float ora_e8m0_decode(uint8_t code)
{
    return (float)ldexp(1.0, (int)code - 127);
}

/* Round y > 0 to the nearest power of two in value (round-to-nearest-even on the
 * significand: below 1.5 rounds down, above 1.5 up, exactly 1.5 goes to the even
 * code), then clamp the code to 0..254 (2^-127 .. 2^127).  y = 0 gives code 0. */
uint8_t ora_e8m0_encode(float y)
{
    if (!(y > 0.0f)) return 0;
    int e;
    double m = frexp((double)y, &e);       /* y = m * 2^e, m in [0.5, 1) */
    double sig = 2.0 * m;                  /* y = sig * 2^(e-1), sig in [1, 2) */
    int k = e - 1;
    if (sig > 1.5) {
        k += 1;
    } else if (sig == 1.5) {
        if (((k + 127) & 1) != 0) k += 1;  /* tie: even code of {k+127, k+128} */
    }
    int code = k + 127;
    if (code < 0) code = 0;
    if (code > 254) code = 254;
    return (uint8_t)code;
}

/* ------------------------------------------------------------------------- */
/* Tensor scale [NV "scaleの導出"]                                              */
/* ------------------------------------------------------------------------- */

static float load_elem(const void* x, int dtype, int64_t i)
{
    if (dtype == ORA_BF16) {
        uint32_t bits = (uint32_t)((const uint16_t*)x)[i] << 16;
        float f;
        memcpy(&f, &bits, 4);
        return f;
    }
    return ((const float*)x)[i];
}

float ora_amax(const void* x, int dtype, int64_t n)
{
    float m = 0.0f;
    for (int64_t i = 0; i < n; ++i) {
        float a = fabsf(load_elem(x, dtype, i));
        if (a > m) m = a;
    }
    return m;
}

/* Global (encode) scale = 6 * 448 / amax, so that the tensor's largest magnitude
 * lands on the largest NVFP4 value 2688.  Reading for the cases the page leaves
 * open: amax = 0 gives 1, and a quotient that overflows binary32 is clamped to
 * FLT_MAX. */
float ora_tensor_scale(float amax)
{
    if (!(amax > 0.0f)) return 1.0f;
    float gs = 2688.0f / amax;
    if (gs > FLT_MAX) gs = FLT_MAX;
    return gs;
}

/* ------------------------------------------------------------------------- */
/* NVFP4 with 1x16 and 16x16 blocks                                            */
/* [NV "scaleの導出", "2D scaling"], [GL "FP4の仕組み"]                           */
/* ------------------------------------------------------------------------- */

/* Block scale from the block's largest magnitude: s = E4M3(fl(fl(bamax*gs)/6)).
 * The page takes the block amax of x2 = x*gs and divides it by 6; rounding is
 * monotone, so amax(fl(x*gs)) = fl(amax(x)*gs). */
static uint8_t nvfp4_block_scale(float bamax, float gs)
{
    float y = (bamax * gs) / 6.0f;
    return ora_e4m3_encode(y);
}

/* One element: v = fl(fl(x*gs)/s) (the page's x2 = x*gs, then x2 / scale), then
 * E2M1.  A block whose scale rounded to zero quantizes every element to a signed
 * zero. */
static uint8_t nvfp4_elem(float x, float gs, float s, int rnd, uint32_t r16)
{
    if (s == 0.0f) return (uint8_t)(signbit(x) ? 8 : 0);
    float t = x * gs;
    float v = t / s;
    return rnd == ORA_SR ? ora_e2m1_sr(v, r16) : ora_e2m1_rtn(v);
}

static void put_nibble(uint8_t* codes, int64_t byte_row_stride, int64_t r, int64_t c, uint8_t nib)
{
    uint8_t* p = codes + r * byte_row_stride + c / 2;
    if (c & 1) *p = (uint8_t)((*p & 0x0F) | (nib << 4));
    else       *p = (uint8_t)((*p & 0xF0) | (nib & 0x0F));
}

/* NVFP4 1x16 on the logical matrix L[lr][lc] = x[lr*sr + lc*sc] (row-wise: sr=cols,
 * sc=1; column-wise: the logical matrix is X^T, sr=1, sc=cols).  Blocks are 16
 * consecutive elements of a logical row.  Outputs: codes[lr][lc/2] (element 2k in
 * the low nibble of byte k, 2k+1 in the high nibble) and scales[lr][lc/16].
 * `row0` is the logical index of the first row handed in (0 for a whole matrix);
 * it only shifts the SR stream index, which is (row0 + r) * lcols + c. */
void ora_quantize_nvfp4_strided(const void* x, int dtype, int64_t lrows, int64_t lcols,
                                int64_t sr, int64_t sc, float gs, int rnd, uint64_t seed,
                                uint32_t stream, int64_t row0, uint8_t* codes, uint8_t* scales)
{
    for (int64_t r = 0; r < lrows; ++r) {
        for (int64_t b = 0; b < lcols / 16; ++b) {
            float bamax = 0.0f;
            for (int64_t k = 0; k < 16; ++k) {
                float a = fabsf(load_elem(x, dtype, r * sr + (b * 16 + k) * sc));
                if (a > bamax) bamax = a;
            }
            uint8_t sc8 = nvfp4_block_scale(bamax, gs);
            float s = ora_e4m3_decode(sc8);
            scales[r * (lcols / 16) + b] = sc8;
            for (int64_t k = 0; k < 16; ++k) {
                int64_t c = b * 16 + k;
                float xv = load_elem(x, dtype, r * sr + c * sc);
                uint32_t r16 = rnd == ORA_SR ? ora_sr_bits16(seed, stream, (uint64_t)((row0 + r) * lcols + c)) : 0u;
                put_nibble(codes, lcols / 2, r, c, nvfp4_elem(xv, gs, s, rnd, r16));
            }
        }
    }
}

void ora_quantize_nvfp4(const void* x, int dtype, int64_t rows, int64_t cols, int colwise,
                        float gs, int rnd, uint64_t seed, uint8_t* codes, uint8_t* scales)
{
    if (colwise)
        ora_quantize_nvfp4_strided(x, dtype, cols, rows, 1, cols, gs, rnd, seed, 1u, 0, codes, scales);
    else
        ora_quantize_nvfp4_strided(x, dtype, rows, cols, cols, 1, gs, rnd, seed, 0u, 0, codes, scales);
}

/* NVFP4 with 16x16 blocks for weights [NV "2D scaling"]: one E4M3 scale per 16x16
 * tile (scales[rows/16][cols/16]), so quantizing W^T gives the transpose of the
 * codes and scales of W.  Round-to-nearest only. */
void ora_quantize_nvfp4_2d(const void* x, int dtype, int64_t rows, int64_t cols, float gs,
                           uint8_t* codes, uint8_t* scales)
{
    for (int64_t br = 0; br < rows / 16; ++br) {
        for (int64_t bc = 0; bc < cols / 16; ++bc) {
            float bamax = 0.0f;
            for (int64_t i = 0; i < 16; ++i)
                for (int64_t j = 0; j < 16; ++j) {
                    float a = fabsf(load_elem(x, dtype, (br * 16 + i) * cols + bc * 16 + j));
                    if (a > bamax) bamax = a;
                }
            uint8_t sc8 = nvfp4_block_scale(bamax, gs);
            float s = ora_e4m3_decode(sc8);
            scales[br * (cols / 16) + bc] = sc8;
            for (int64_t i = 0; i < 16; ++i)
                for (int64_t j = 0; j < 16; ++j) {
                    int64_t r = br * 16 + i, c = bc * 16 + j;
                    float xv = load_elem(x, dtype, r * cols + c);
                    put_nibble(codes, cols / 2, r, c, nvfp4_elem(xv, gs, s, ORA_RTN, 0u));
                }
        }
    }
}

/* ------------------------------------------------------------------------- */
/* MXFP4: 32 elements + one E8M0 scale [GL "FP4の仕組み"], [F6]                  */
/* ------------------------------------------------------------------------- */

/* Reading: the block scale is amax/6 (the block's largest magnitude maps to about
 * 6) rounded to a power of two with round-to-nearest-even; elements are divided by
 * that power of two (one rounding, exact unless the result is subnormal) and
 * rounded onto E2M1 (RTN, or SR with stream 0).  No tensor scale. */
void ora_quantize_mxfp4(const void* x, int dtype, int64_t rows, int64_t cols, int rnd,
                        uint64_t seed, uint8_t* codes, uint8_t* scales)
{
    for (int64_t r = 0; r < rows; ++r) {
        for (int64_t b = 0; b < cols / 32; ++b) {
            float bamax = 0.0f;
            for (int64_t k = 0; k < 32; ++k) {
                float a = fabsf(load_elem(x, dtype, r * cols + b * 32 + k));
                if (a > bamax) bamax = a;
            }
            uint8_t e8 = ora_e8m0_encode(bamax / 6.0f);
            scales[r * (cols / 32) + b] = e8;
            int k_exp = (int)e8 - 127;
            for (int64_t k = 0; k < 32; ++k) {
                int64_t c = b * 32 + k;
                float v = ldexpf(load_elem(x, dtype, r * cols + c), -k_exp);
                uint8_t nib;
                if (rnd == ORA_SR)
                    nib = ora_e2m1_sr(v, ora_sr_bits16(seed, 0u, (uint64_t)(r * cols + c)));
                else
                    nib = ora_e2m1_rtn(v);
                put_nibble(codes, cols / 2, r, c, nib);
            }
        }
    }
}

/* ------------------------------------------------------------------------- */
/* IF4: per-block FP4 or INT4 [IF "2. 提案手法：IF4"]                           */
/* ------------------------------------------------------------------------- */

/* Each 16-element row block is quantized twice with the NVFP4 scale s:
 *  - FP4: r_i = E2M1_RTN(v_i);
 *  - INT4 with the 6/7 rule: q_i = clamp(rint(fl(v_i * fl(7/6))), -7, 7), restored
 *    as r_i = fl(q_i * fl(6/7)), so both candidates span 0..6;
 * and the candidate with the lower squared error sum_i (v_i - r_i)^2 is kept.
 * Readings: the error is taken in the scaled domain (a common factor per block),
 * summed for i = 0..15 in order, each term added with one fused multiply-add
 * e = fma(d, d, e) after d = fl(v_i - r_i); INT4 wins only if strictly lower.
 * The choice is flagged in the scale byte's sign bit (set = INT4); INT4 codes are
 * two's-complement nibbles.  A zero-scale block is FP4 with signed zeros. */
void ora_quantize_if4(const void* x, int dtype, int64_t rows, int64_t cols, float gs,
                      uint8_t* codes, uint8_t* scales)
{
    const float c76 = 7.0f / 6.0f;
    const float c67 = 6.0f / 7.0f;
    for (int64_t r = 0; r < rows; ++r) {
        for (int64_t b = 0; b < cols / 16; ++b) {
            float xv[16], v[16];
            float bamax = 0.0f;
            for (int k = 0; k < 16; ++k) {
                xv[k] = load_elem(x, dtype, r * cols + b * 16 + k);
                float a = fabsf(xv[k]);
                if (a > bamax) bamax = a;
            }
            uint8_t sc8 = nvfp4_block_scale(bamax, gs);
            float s = ora_e4m3_decode(sc8);
            uint8_t fp_nib[16], int_nib[16];
            float e_fp = 0.0f, e_int = 0.0f;
            for (int k = 0; k < 16; ++k) {
                if (s == 0.0f) {
                    fp_nib[k] = (uint8_t)(signbit(xv[k]) ? 8 : 0);
                    int_nib[k] = 0;
                    continue;
                }
                float t = xv[k] * gs;
                v[k] = t / s;
                fp_nib[k] = ora_e2m1_rtn(v[k]);
                float rf = ora_e2m1_decode(fp_nib[k]);
                float w = v[k] * c76;
                float q = rintf(w);
                if (q > 7.0f) q = 7.0f;
                if (q < -7.0f) q = -7.0f;
                float ri = q * c67;
                int_nib[k] = (uint8_t)(((int)q) & 0xF);
                float dfp = v[k] - rf;
                float dint = v[k] - ri;
                e_fp = fmaf(dfp, dfp, e_fp);
                e_int = fmaf(dint, dint, e_int);
            }
            int use_int = (s != 0.0f) && (e_int < e_fp);
            scales[r * (cols / 16) + b] = (uint8_t)(sc8 | (use_int ? 0x80 : 0));
            for (int k = 0; k < 16; ++k)
                put_nibble(codes, cols / 2, r, b * 16 + k, use_int ? int_nib[k] : fp_nib[k]);
        }
    }
}

/* INT4 restore of one two's-complement nibble under the 6/7 rule. */
float ora_int4_decode(uint8_t nibble)
{
    int q = (nibble & 8) ? (int)(nibble & 0xF) - 16 : (int)(nibble & 0xF);
    return (float)q * (6.0f / 7.0f);
}

/* ------------------------------------------------------------------------- */
/* Dequantization                                                              */
/* ------------------------------------------------------------------------- */

static uint8_t get_nibble(const uint8_t* codes, int64_t cols, int64_t r, int64_t c)
{
    uint8_t byte = codes[r * (cols / 2) + c / 2];
    return (c & 1) ? (uint8_t)(byte >> 4) : (uint8_t)(byte & 0xF);
}

/* x_hat = fl(fl(r*s)/gs): the element value times its block scale, divided by the
 * tensor's encode scale.  fmt: 0 NVFP4 1x16, 1 NVFP4 16x16, 3 IF4 (flag in scale
 * bit 7 selects the INT4 restore).  MXFP4 (fmt 2): x_hat = r * 2^(code-127). */
void ora_dequantize(int fmt, const uint8_t* codes, const uint8_t* scales, float gs,
                    int64_t rows, int64_t cols, float* y)
{
    for (int64_t r = 0; r < rows; ++r) {
        for (int64_t c = 0; c < cols; ++c) {
            uint8_t nib = get_nibble(codes, cols, r, c);
            float out;
            if (fmt == 2) {
                uint8_t e8 = scales[r * (cols / 32) + c / 32];
                out = ldexpf(ora_e2m1_decode(nib), (int)e8 - 127);
            } else {
                uint8_t sc8 = (fmt == 1) ? scales[(r / 16) * (cols / 16) + c / 16]
                                         : scales[r * (cols / 16) + c / 16];
                float s = ora_e4m3_decode((uint8_t)(sc8 & 0x7F));
                float rv = (fmt == 3 && (sc8 & 0x80)) ? ora_int4_decode(nib) : ora_e2m1_decode(nib);
                float p = rv * s;
                out = p / gs;
            }
            y[r * cols + c] = out;
        }
    }
}

/* ------------------------------------------------------------------------- */
/* MX FP6 [F6 "FP6で隣り合う値の間隔を見てみる", "量子化と6bitの保存"]             */
/* ------------------------------------------------------------------------- */

/* The two six-bit formats of the OCP MX specification as the page describes them:
 * sign, then exponent and mantissa bits; fmt 0 = E2M3 (bias 1, largest 7.5), fmt 1 =
 * E3M2 (bias 3, largest 28, smallest step 0.0625); exponent field 0 holds the
 * subnormals; no Inf or NaN codes. */
float ora_fp6_decode(int fmt, uint8_t code)
{
    const int ebits = fmt ? 3 : 2, mbits = 5 - ebits, bias = fmt ? 3 : 1;
    const int s = (code >> 5) & 1, e = (code >> mbits) & ((1 << ebits) - 1), m = code & ((1 << mbits) - 1);
    double v = (e == 0) ? ldexp((double)m, 1 - bias - mbits)
                        : ldexp((double)((1 << mbits) + m), e - bias - mbits);
    return (float)(s ? -v : v);
}

/* Reading: round to the nearest of the 32 magnitudes, ties to the even code (as for
 * E2M1), saturating at the largest; the sign bit is copied (so -0 and tiny negative
 * values give 0x20). */
uint8_t ora_fp6_rtn(int fmt, float v)
{
    const double a = fabs((double)v);
    const uint8_t sign = signbit(v) ? 0x20 : 0;
    /* at or beyond the largest magnitude: saturate (the distances below would absorb
     * the difference between the two largest values for huge inputs) */
    if (a >= (double)ora_fp6_decode(fmt, 31)) return (uint8_t)(31 | sign);
    int best = 0;
    double bestd = INFINITY;
    for (int c = 0; c < 32; ++c) {
        const double d = fabs(a - (double)ora_fp6_decode(fmt, (uint8_t)c));
        if (d < bestd || (d == bestd && (c & 1) == 0)) {
            best = c;
            bestd = d;
        }
    }
    return (uint8_t)(best | sign);
}

/* Four six-bit codes per three bytes [F6 "量子化と6bitの保存"]: code j of a group in
 * bits 6j .. 6j+5 of the little-endian 24-bit word the three bytes form.  A row of c
 * elements takes 3c/4 bytes. */
static void put6(uint8_t* codes, int64_t row_bytes, int64_t r, int64_t c, uint8_t code)
{
    uint8_t* g = codes + r * row_bytes + (c / 4) * 3;
    uint32_t w = (uint32_t)g[0] | ((uint32_t)g[1] << 8) | ((uint32_t)g[2] << 16);
    const int sh = 6 * (int)(c % 4);
    w = (w & ~(0x3Fu << sh)) | ((uint32_t)(code & 0x3F) << sh);
    g[0] = (uint8_t)w;
    g[1] = (uint8_t)(w >> 8);
    g[2] = (uint8_t)(w >> 16);
}

static uint8_t get6(const uint8_t* codes, int64_t row_bytes, int64_t r, int64_t c)
{
    const uint8_t* g = codes + r * row_bytes + (c / 4) * 3;
    const uint32_t w = (uint32_t)g[0] | ((uint32_t)g[1] << 8) | ((uint32_t)g[2] << 16);
    return (uint8_t)((w >> (6 * (int)(c % 4))) & 0x3F);
}

/* MX FP6: blocks of 32 with one E8M0 scale, as MXFP4 with the format's largest value
 * in place of 6: scale code E8M0_RNE(fl(bamax / max)), elements x * 2^(127 - code)
 * (one rounding) rounded as ora_fp6_rtn.  codes [rows][3 cols / 4], scales [rows][cols/32]. */
void ora_quantize_mxfp6(const void* x, int dtype, int64_t rows, int64_t cols, int fmt, uint8_t* codes,
                        uint8_t* scales)
{
    const float maxv = fmt ? 28.0f : 7.5f;
    for (int64_t r = 0; r < rows; ++r) {
        for (int64_t b = 0; b < cols / 32; ++b) {
            float bamax = 0.0f;
            for (int64_t k = 0; k < 32; ++k) {
                float a = fabsf(load_elem(x, dtype, r * cols + b * 32 + k));
                if (a > bamax) bamax = a;
            }
            const uint8_t e8 = ora_e8m0_encode(bamax / maxv);
            scales[r * (cols / 32) + b] = e8;
            for (int64_t k = 0; k < 32; ++k) {
                const int64_t c = b * 32 + k;
                const float v = ldexpf(load_elem(x, dtype, r * cols + c), 127 - (int)e8);
                put6(codes, cols / 4 * 3, r, c, ora_fp6_rtn(fmt, v));
            }
        }
    }
}

/* x_hat = fp6(code) * 2^(scale - 127), one rounding. */
void ora_dequantize_mxfp6(int fmt, const uint8_t* codes, const uint8_t* scales, int64_t rows, int64_t cols,
                          float* y)
{
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t c = 0; c < cols; ++c)
            y[r * cols + c] = ldexpf(ora_fp6_decode(fmt, get6(codes, cols / 4 * 3, r, c)),
                                     (int)scales[r * (cols / 32) + c / 32] - 127);
}

/* ------------------------------------------------------------------------- */
/* FP4 GEMM consumer [NV "NVFP4フロー図"], [GL "FP4による推論と学習"]             */
/* ------------------------------------------------------------------------- */

/* The products that follow quantization (forward, data-gradient and weight-gradient
 * GEMMs) take two operands quantized along the reduction dimension K and accumulate
 * in higher precision.  Reading: both operands are row-wise MXFP4 along K, A is
 * [m][k] and B is [n][k], and
 *     C[i][j] = sum_k a(i,k) * b(j,k),   a(i,k) = E2M1(nibble) * 2^(e8m0 - 127).
 * Each product and the running sum (k ascending) are binary64; with E2M1 values of at
 * most two significant bits, the products are exact and so is the sum while the
 * operands' exponents stay within binary64's 53-bit window, which holds for the
 * scales quantization produces.  cabs[i][j] = sum_k |a(i,k) * b(j,k)| is returned
 * for error bounds.  Row strides: codes k/2 bytes, scales k/32 bytes. */
void ora_gemm_mxfp4(const uint8_t* a_codes, const uint8_t* a_scales, const uint8_t* b_codes,
                    const uint8_t* b_scales, int64_t m, int64_t n, int64_t k, double* c, double* cabs)
{
    for (int64_t i = 0; i < m; ++i) {
        for (int64_t j = 0; j < n; ++j) {
            double acc = 0.0, mag = 0.0;
            for (int64_t t = 0; t < k; ++t) {
                double av = ldexp((double)ora_e2m1_decode(get_nibble(a_codes, k, i, t)),
                                  (int)a_scales[i * (k / 32) + t / 32] - 127);
                double bv = ldexp((double)ora_e2m1_decode(get_nibble(b_codes, k, j, t)),
                                  (int)b_scales[j * (k / 32) + t / 32] - 127);
                acc += av * bv;
                mag += fabs(av * bv);
            }
            c[i * n + j] = acc;
            if (cabs) cabs[i * n + j] = mag;
        }
    }
}

/* The same product over two row-wise NVFP4 1x16 operands [NV "NVFP4フロー図"], whose
 * dequantized values are r * s / gs (r the E2M1 value, s the block's E4M3 scale, gs
 * the operand's tensor encode scale) [NV "scaleの導出"]:
 *     C[i][j] = (sum_t (r_a s_a)(r_b s_b)) / (gs_a * gs_b).
 * r * s has at most six significant bits, so every product and (for the scales that
 * quantization produces) the binary64 sum are exact; the one division by the binary64
 * product gs_a * gs_b (exact: two 24-bit significands) rounds once.  cabs is the sum of
 * |products| over the same divisor.  Scale row strides: k/16 bytes. */
/* One element of a GEMM operand, r * s in binary64 (exact): an E2M1 value times its
 * block's E4M3 scale or, in an IF4 operand's INT4 block (scale bit 7 set
 * [IF "2. 提案手法：IF4"]), the 6/7-rule restore fl(q * fl(6/7)) times the scale. */
static double gemm_elem(const uint8_t* codes, uint8_t scale, int if4, int64_t k, int64_t row, int64_t t)
{
    const uint8_t nib = get_nibble(codes, k, row, t);
    if (if4 && (scale & 0x80))
        return (double)ora_int4_decode(nib) * (double)ora_e4m3_decode((uint8_t)(scale & 0x7F));
    return (double)ora_e2m1_decode(nib) * (double)ora_e4m3_decode(scale);
}

void ora_gemm_nvfp4(const uint8_t* a_codes, const uint8_t* a_scales, float gs_a, const uint8_t* b_codes,
                    const uint8_t* b_scales, float gs_b, int64_t m, int64_t n, int64_t k, int flags,
                    double* c, double* cabs)
{
    /* flags bit 0 / bit 1: A / B holds one scale per 16x16 tile [NV "2D scaling"], so
     * element (i, t) takes the scale of tile (i / 16, t / 16) instead of block (i, t / 16);
     * bit 2 / bit 3: A / B is IF4 (1x16 blocks whose flagged scales mark INT4 blocks). */
    const double g = (double)gs_a * (double)gs_b;
    const int if4_a = (flags >> 2) & 1, if4_b = (flags >> 3) & 1;
    for (int64_t i = 0; i < m; ++i) {
        const int64_t sa = (flags & 1) ? i / 16 : i;
        for (int64_t j = 0; j < n; ++j) {
            const int64_t sb = (flags & 2) ? j / 16 : j;
            double acc = 0.0, mag = 0.0;
            for (int64_t t = 0; t < k; ++t) {
                double av = gemm_elem(a_codes, a_scales[sa * (k / 16) + t / 16], if4_a, k, i, t);
                double bv = gemm_elem(b_codes, b_scales[sb * (k / 16) + t / 16], if4_b, k, j, t);
                acc += av * bv;
                mag += fabs(av * bv);
            }
            c[i * n + j] = acc / g;
            if (cabs) cabs[i * n + j] = mag / g;
        }
    }
}

/* ------------------------------------------------------------------------- */
/* Random Hadamard transform [NV "ランダムアダマール変換"]                         */
/* ------------------------------------------------------------------------- */

/* Sylvester Hadamard entry: H[i][t] = (-1)^popcount(i & t), 128 x 128, H H^T = 128 I. */
int ora_hadamard_entry(int i, int t)
{
    int p = 0;
    for (int b = i & t; b; b >>= 1) p ^= (b & 1);
    return p ? -1 : 1;
}

static int sign_of(const uint32_t signs[4], int t)
{
    return ((signs[t >> 5] >> (t & 31)) & 1u) ? -1 : 1;
}

/* Along the token (row) dimension, per chunk of 128 rows, with R = S*H/sqrt(128):
 *   forward  B = R^T A:  B[128c+i][j] = (1/sqrt(128)) * sum_t H[i][t] s_t A[128c+t][j]
 *   inverse  A = R B:    A[128c+t][j] = (1/sqrt(128)) * s_t * sum_i H[t][i] B[128c+i][j]
 * Products and sums in binary64 (t or i ascending), one rounding to binary32 at the
 * end.  R R^T = I, so the inverse undoes the forward transform. */
void ora_rht(const void* x, int dtype, int64_t rows, int64_t cols, const uint32_t signs[4],
             int inverse, float* y)
{
    const double kappa = 1.0 / sqrt(128.0);
    for (int64_t c0 = 0; c0 < rows; c0 += 128) {
        for (int i = 0; i < 128; ++i) {
            for (int64_t j = 0; j < cols; ++j) {
                double acc = 0.0;
                for (int t = 0; t < 128; ++t) {
                    double a = (double)load_elem(x, dtype, (c0 + t) * cols + j);
                    double h = (double)ora_hadamard_entry(i, t);
                    if (!inverse) h *= (double)sign_of(signs, t);
                    acc += h * a;
                }
                if (inverse) acc *= (double)sign_of(signs, i);
                y[(c0 + i) * cols + j] = (float)(acc * kappa);
            }
        }
    }
}

/* The RHT of one column j only, rows [0, rows): y[i] for the chosen column, so
 * that sampled checks at full size need not transform the whole matrix. */
void ora_rht_column(const void* x, int dtype, int64_t rows, int64_t cols, int64_t j,
                    const uint32_t signs[4], float* y)
{
    const double kappa = 1.0 / sqrt(128.0);
    for (int64_t c0 = 0; c0 < rows; c0 += 128) {
        for (int i = 0; i < 128; ++i) {
            double acc = 0.0;
            for (int t = 0; t < 128; ++t) {
                double a = (double)load_elem(x, dtype, (c0 + t) * cols + j);
                acc += (double)ora_hadamard_entry(i, t) * (double)sign_of(signs, t) * a;
            }
            y[c0 + i] = (float)(acc * kappa);
        }
    }
}

/* ------------------------------------------------------------------------- */
/* The glossary's block-size comparison [GL "FP4の仕組み"]                       */
/* ------------------------------------------------------------------------- */

/* Plain per-block scaling as the glossary describes it: scale = amax/6 kept as a
 * binary32 value (no E4M3/E8M0 rounding), each |x|/scale goes to the nearest E2M1
 * magnitude (ties to the smaller magnitude), and x_hat = sign(x) * g * scale.
 * A zero block reconstructs to zero.  n must be a multiple of `block`. */
void ora_plain_block_roundtrip(const float* x, int64_t n, int64_t block, float* y)
{
    for (int64_t b0 = 0; b0 < n; b0 += block) {
        float amax = 0.0f;
        for (int64_t k = 0; k < block; ++k)
            if (fabsf(x[b0 + k]) > amax) amax = fabsf(x[b0 + k]);
        float scale = amax / 6.0f;
        for (int64_t k = 0; k < block; ++k) {
            float xv = x[b0 + k];
            if (scale == 0.0f) {
                y[b0 + k] = 0.0f;
                continue;
            }
            float q = fabsf(xv) / scale;
            int best = 0;
            float best_d = fabsf(q - E2M1_MAG[0]);
            for (int c = 1; c < 8; ++c) {
                float d = fabsf(q - E2M1_MAG[c]);
                if (d < best_d) {
                    best = c;
                    best_d = d;
                }
            }
            float sgn = xv > 0.0f ? 1.0f : (xv < 0.0f ? -1.0f : 0.0f);
            y[b0 + k] = E2M1_MAG[best] * sgn * scale;
        }
    }
}

/* ------------------------------------------------------------------------- */
/* Block-format variants [IF "1. 背景と問題点", "2. 提案手法：IF4", "3. 主要な貢献"] */
/* ------------------------------------------------------------------------- */

/* The variants the IF explainer compares IF4 against, and its 3- and 6-bit
 * extensions, all with NVFP4's two-level scaling on 16-element row blocks: an FP32
 * tensor encode scale gs = fl(448 * M / amax) and an E4M3 block scale
 * s = E4M3(fl(fl(bamax * gs) / M)), where M is the block maximum the format maps the
 * block's largest magnitude to.  Elements are v = fl(fl(x * gs) / s).  Readings (the
 * page names the formats and their key property, not every constant):
 *   ORA_VAR_46     Four Over Six: NVFP4 with the block maximum 4 instead of 6 (M = 4);
 *                  E2M1 elements, so the values +-6 are never produced.
 *   ORA_VAR_NVINT4 NVFP4 scaling with INT4 elements: M = 7, q = clamp(RNE(v), -7, 7),
 *                  two's-complement nibbles.
 *   ORA_VAR_IF3    per block the better of FP3 (E2M0: 0, 1, 2, 4; M = 4) and INT3
 *                  scaled by the IF4 rule: q = clamp(RNE(fl(v * fl(3/4))), -3, 3),
 *                  restored as fl(q * fl(4/3)).
 *   ORA_VAR_IF4    the same generalisation at 4 bits: E2M1 (M = 6) or INT4 with 7/6;
 *                  it must equal ora_quantize_if4.
 *   ORA_VAR_IF6    FP6 E2M3 (M = 7.5) or INT6 with fl(31/7.5), restored with fl(7.5/31).
 * The choice, the error sums and the flag (bit 7 of the scale byte, set = INT) are
 * IF4's.  Code layouts: 4-bit formats as NVFP4 (two per byte); IF3 packs eight 3-bit
 * codes into three bytes (code j at bits 3j..3j+2 of the little-endian 24-bit word;
 * FP3 code = sign bit 2, exponent bits 1..0; INT3 two's complement); IF6 packs four
 * 6-bit codes into three bytes as MX FP6 does (FP6 E2M3 codes, INT6 two's complement). */

/* FP3 E2M0 (bias 1, exponent field 0 = zero): magnitudes 0, 1, 2, 4. */
float ora_fp3_decode(uint8_t code)
{
    static const float mag[4] = {0.0f, 1.0f, 2.0f, 4.0f};
    float m = mag[code & 3];
    return (code & 4) ? -m : m;
}

/* Nearest FP3 magnitude, ties to the even code, saturating at 4; sign copied. */
uint8_t ora_fp3_rtn(float v)
{
    double a = fabs((double)v);
    int best = 0;
    double bd = a;
    for (int c = 1; c < 4; ++c) {
        double d = fabs(a - (double)ora_fp3_decode((uint8_t)c));
        if (d < bd || (d == bd && (c & 1) == 0)) {
            best = c;
            bd = d;
        }
    }
    if (a >= 4.0) best = 3;
    return (uint8_t)(best | (signbit(v) ? 4 : 0));
}

typedef struct {
    int bits;        /* code width */
    float m;         /* block maximum M */
    int has_fp, has_int;
    int qmax;        /* INT range +-qmax */
    int int_direct;  /* 1: INT codes round v itself (NVINT4); 0: fl(v * c), restored fl(q * cinv) */
    float c, cinv;
} ora_variant;

static ora_variant variant_of(int var)
{
    ora_variant d;
    memset(&d, 0, sizeof d);
    switch (var) {
    case ORA_VAR_46:     d.bits = 4; d.m = 4.0f; d.has_fp = 1; break;
    case ORA_VAR_NVINT4: d.bits = 4; d.m = 7.0f; d.has_int = 1; d.qmax = 7; d.int_direct = 1; break;
    case ORA_VAR_IF3:    d.bits = 3; d.m = 4.0f; d.has_fp = d.has_int = 1; d.qmax = 3;
                         d.c = 3.0f / 4.0f; d.cinv = 4.0f / 3.0f; break;
    case ORA_VAR_IF4:    d.bits = 4; d.m = 6.0f; d.has_fp = d.has_int = 1; d.qmax = 7;
                         d.c = 7.0f / 6.0f; d.cinv = 6.0f / 7.0f; break;
    default:             d.bits = 6; d.m = 7.5f; d.has_fp = d.has_int = 1; d.qmax = 31;
                         d.c = 31.0f / 7.5f; d.cinv = 7.5f / 31.0f; break;
    }
    return d;
}

static uint8_t fp_rtn_bits(int bits, float v)
{
    if (bits == 3) return ora_fp3_rtn(v);
    if (bits == 4) return ora_e2m1_rtn(v);
    return ora_fp6_rtn(0, v);
}

static float fp_decode_bits(int bits, uint8_t code)
{
    if (bits == 3) return ora_fp3_decode(code);
    if (bits == 4) return ora_e2m1_decode(code);
    return ora_fp6_decode(0, code);
}

/* Code c of element j of a row, in the row's packed bytes. */
static void put_code(uint8_t* row, int bits, int64_t j, uint8_t code)
{
    if (bits == 4) {
        uint8_t* p = row + j / 2;
        *p = (j & 1) ? (uint8_t)((*p & 0x0F) | (code << 4)) : (uint8_t)((*p & 0xF0) | (code & 0x0F));
        return;
    }
    const int per = bits == 3 ? 8 : 4;                    /* codes per three bytes */
    uint8_t* g = row + (j / per) * 3;
    uint32_t w = (uint32_t)g[0] | ((uint32_t)g[1] << 8) | ((uint32_t)g[2] << 16);
    const int sh = bits * (int)(j % per);
    const uint32_t mask = (1u << bits) - 1u;
    w = (w & ~(mask << sh)) | ((uint32_t)(code & mask) << sh);
    g[0] = (uint8_t)w;
    g[1] = (uint8_t)(w >> 8);
    g[2] = (uint8_t)(w >> 16);
}

static uint8_t get_code(const uint8_t* row, int bits, int64_t j)
{
    if (bits == 4) return (uint8_t)((j & 1) ? row[j / 2] >> 4 : row[j / 2] & 0x0F);
    const int per = bits == 3 ? 8 : 4;
    const uint8_t* g = row + (j / per) * 3;
    const uint32_t w = (uint32_t)g[0] | ((uint32_t)g[1] << 8) | ((uint32_t)g[2] << 16);
    return (uint8_t)((w >> (bits * (int)(j % per))) & ((1u << bits) - 1u));
}

int64_t ora_variant_row_bytes(int var, int64_t cols)
{
    return cols * variant_of(var).bits / 8;
}

float ora_variant_tensor_scale(int var, float amax)
{
    if (!(amax > 0.0f)) return 1.0f;
    float gs = (448.0f * variant_of(var).m) / amax;
    if (gs > FLT_MAX) gs = FLT_MAX;
    return gs;
}

/* INT restore of a stored INT code. */
static float int_value(const ora_variant* d, uint8_t code)
{
    const int sh = 32 - d->bits;
    const int q = (int)((uint32_t)code << sh) >> sh;      /* sign-extend the code */
    return d->int_direct ? (float)q : (float)q * d->cinv;
}

void ora_quantize_variant(const void* x, int dtype, int64_t rows, int64_t cols, int var, float gs,
                          uint8_t* codes, uint8_t* scales)
{
    const ora_variant d = variant_of(var);
    const int64_t rb = cols * d.bits / 8;
    for (int64_t r = 0; r < rows; ++r) {
        for (int64_t b = 0; b < cols / 16; ++b) {
            float xv[16], v[16];
            float bamax = 0.0f;
            for (int k = 0; k < 16; ++k) {
                xv[k] = load_elem(x, dtype, r * cols + b * 16 + k);
                if (fabsf(xv[k]) > bamax) bamax = fabsf(xv[k]);
            }
            const uint8_t sc8 = ora_e4m3_encode((bamax * gs) / d.m);
            const float s = ora_e4m3_decode(sc8);
            uint8_t fpc[16], intc[16];
            float e_fp = 0.0f, e_int = 0.0f;
            for (int k = 0; k < 16; ++k) {
                if (s == 0.0f) {                               /* a zero block: signed zeros */
                    fpc[k] = d.has_fp ? fp_rtn_bits(d.bits, signbit(xv[k]) ? -0.0f : 0.0f) : 0;
                    intc[k] = 0;
                    continue;
                }
                v[k] = (xv[k] * gs) / s;
                if (d.has_fp) {
                    fpc[k] = fp_rtn_bits(d.bits, v[k]);
                    const float df = v[k] - fp_decode_bits(d.bits, fpc[k]);
                    e_fp = fmaf(df, df, e_fp);
                }
                if (d.has_int) {
                    float q = rintf(d.int_direct ? v[k] : v[k] * d.c);
                    if (q > (float)d.qmax) q = (float)d.qmax;
                    if (q < -(float)d.qmax) q = -(float)d.qmax;
                    intc[k] = (uint8_t)((int)q & ((1 << d.bits) - 1));
                    const float di = v[k] - (d.int_direct ? q : q * d.cinv);
                    e_int = fmaf(di, di, e_int);
                }
            }
            const int use_int = d.has_int && (!d.has_fp || (s != 0.0f && e_int < e_fp));
            scales[r * (cols / 16) + b] = (uint8_t)(sc8 | (d.has_fp && use_int ? 0x80 : 0));
            for (int k = 0; k < 16; ++k)
                put_code(codes + r * rb, d.bits, b * 16 + k, use_int ? intc[k] : fpc[k]);
        }
    }
}

/* x_hat = fl(fl(r * s) / gs): r the FP value, or the INT restore for flagged blocks
 * (every block for NVINT4). */
void ora_dequantize_variant(int var, const uint8_t* codes, const uint8_t* scales, float gs, int64_t rows,
                            int64_t cols, float* y)
{
    const ora_variant d = variant_of(var);
    const int64_t rb = cols * d.bits / 8;
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t c = 0; c < cols; ++c) {
            const uint8_t sc8 = scales[r * (cols / 16) + c / 16];
            const float s = ora_e4m3_decode((uint8_t)(sc8 & 0x7F));
            const uint8_t code = get_code(codes + r * rb, d.bits, c);
            const int is_int = !d.has_fp || (sc8 & 0x80);
            const float rv = is_int ? int_value(&d, code) : fp_decode_bits(d.bits, code);
            const float p = rv * s;
            y[r * cols + c] = p / gs;
        }
}

/* ------------------------------------------------------------------------- */
/* Array forms of the element codecs (plain loops, for the tests' sweeps)      */
/* ------------------------------------------------------------------------- */

void ora_e2m1_rtn_array(const float* v, int64_t n, uint8_t* out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = ora_e2m1_rtn(v[i]);
}

void ora_e2m1_sr_array(const float* v, const uint32_t* r16, int64_t n, uint8_t* out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = ora_e2m1_sr(v[i], r16[i]);
}

void ora_e4m3_encode_array(const float* y, int64_t n, uint8_t* out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = ora_e4m3_encode(y[i]);
}

void ora_e8m0_encode_array(const float* y, int64_t n, uint8_t* out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = ora_e8m0_encode(y[i]);
}

void ora_sr_bits16_array(uint64_t seed, uint32_t stream, const uint64_t* idx, int64_t n, uint32_t* out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = ora_sr_bits16(seed, stream, idx[i]);
}
