/*
 * oracle_driver.c -- calls every function of the CPU oracle on small inputs, including
 * ragged and degenerate ones (all zeros, signed zeros, single blocks, huge and tiny
 * magnitudes), so that a build with AddressSanitizer and UndefinedBehaviorSanitizer
 * (-fsanitize=address,undefined -fno-sanitize-recover=all) sees every code path of the
 * oracle touch only the memory it is given.  Buffers are allocated at their exact sizes
 * so an overrun is caught.  Exit status 0 means every call returned and the few
 * invariants checked here held; a sanitizer report aborts with a non-zero status.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "fp4q_oracle.h"

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;

static uint32_t next_u32(void)
{
    rng_state ^= rng_state << 13;
    rng_state ^= rng_state >> 7;
    rng_state ^= rng_state << 17;
    return (uint32_t)(rng_state >> 16);
}

static float next_normal(void)
{
    /* sum of uniforms: roughly normal, enough to exercise the code paths */
    float s = 0.0f;
    for (int i = 0; i < 12; ++i) s += (float)(next_u32() & 0xFFFFFF) / 16777216.0f;
    return s - 6.0f;
}

static void* xmalloc(size_t n)
{
    void* p = malloc(n ? n : 1);
    if (!p) {
        fprintf(stderr, "out of memory\n");
        exit(2);
    }
    return p;
}

static float* make_f32(int64_t n, float gain, int kind)
{
    float* x = xmalloc((size_t)n * sizeof(float));
    for (int64_t i = 0; i < n; ++i) {
        switch (kind) {
        case 0: x[i] = next_normal() * gain; break;
        case 1: x[i] = 0.0f; break;
        case 2: x[i] = (i & 1) ? -0.0f : 0.0f; break;
        case 3: x[i] = (i % 7 == 0) ? 3.0e38f : 1.0e-30f * next_normal(); break;
        default: x[i] = (float)(i % 13) - 6.0f; break;
        }
    }
    return x;
}

static uint16_t* to_bf16(const float* x, int64_t n)
{
    uint16_t* b = xmalloc((size_t)n * sizeof(uint16_t));
    for (int64_t i = 0; i < n; ++i) {
        uint32_t u;
        memcpy(&u, &x[i], 4);
        b[i] = (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
    }
    return b;
}

static int failures = 0;

static void expect(int cond, const char* what)
{
    if (!cond) {
        fprintf(stderr, "FAILED: %s\n", what);
        ++failures;
    }
}

/* Every 1x16 / 16x16 / 1x32 quantizer and the dequantizer on one input. */
static void quantizers(const void* x, int dtype, int64_t rows, int64_t cols)
{
    const int64_t n = rows * cols;
    const float amax = ora_amax(x, dtype, n);
    const float gs = ora_tensor_scale(amax);
    float* y = xmalloc((size_t)n * sizeof(float));

    if (cols % 16 == 0) {
        for (int rnd = 0; rnd < 2; ++rnd) {
            uint8_t* codes = xmalloc((size_t)(n / 2));
            uint8_t* scales = xmalloc((size_t)(n / 16));
            ora_quantize_nvfp4(x, dtype, rows, cols, 0, gs, rnd, 7u, codes, scales);
            ora_dequantize(0, codes, scales, gs, rows, cols, y);
            for (int64_t i = 0; i < n; ++i) expect(!isnan(y[i]), "nvfp4 dequant finite");
            ora_quantize_nvfp4_strided(x, dtype, rows > 1 ? rows - 1 : rows, cols, cols, 1, gs, rnd, 7u, 0u, 0,
                                       codes, scales);
            free(codes);
            free(scales);
        }
        uint8_t* codes = xmalloc((size_t)(n / 2));
        uint8_t* scales = xmalloc((size_t)(n / 16));
        ora_quantize_if4(x, dtype, rows, cols, gs, codes, scales);
        ora_dequantize(3, codes, scales, gs, rows, cols, y);
        free(codes);
        free(scales);
    }
    if (rows % 16 == 0) {
        for (int rnd = 0; rnd < 2; ++rnd) {
            uint8_t* codes = xmalloc((size_t)(n / 2));
            uint8_t* scales = xmalloc((size_t)(n / 16));
            ora_quantize_nvfp4(x, dtype, rows, cols, 1, gs, rnd, 9u, codes, scales);
            ora_dequantize(0, codes, scales, gs, cols, rows, y);
            free(codes);
            free(scales);
        }
    }
    if (rows % 16 == 0 && cols % 16 == 0) {
        uint8_t* codes = xmalloc((size_t)(n / 2));
        uint8_t* scales = xmalloc((size_t)(n / 256));
        ora_quantize_nvfp4_2d(x, dtype, rows, cols, gs, codes, scales);
        ora_dequantize(1, codes, scales, gs, rows, cols, y);
        free(codes);
        free(scales);
    }
    if (cols % 32 == 0) {
        for (int rnd = 0; rnd < 2; ++rnd) {
            uint8_t* codes = xmalloc((size_t)(n / 2));
            uint8_t* scales = xmalloc((size_t)(n / 32));
            ora_quantize_mxfp4(x, dtype, rows, cols, rnd, 11u, codes, scales);
            ora_dequantize(2, codes, scales, 1.0f, rows, cols, y);
            free(codes);
            free(scales);
        }
        for (int fmt = 0; fmt < 2; ++fmt) {
            uint8_t* codes = xmalloc((size_t)(n / 4 * 3));
            uint8_t* scales = xmalloc((size_t)(n / 32));
            ora_quantize_mxfp6(x, dtype, rows, cols, fmt, codes, scales);
            ora_dequantize_mxfp6(fmt, codes, scales, rows, cols, y);
            free(codes);
            free(scales);
        }
    }
    if (rows % 128 == 0) {
        uint32_t signs[4];
        ora_rht_signs(5u, signs);
        float* b = xmalloc((size_t)n * sizeof(float));
        float* a = xmalloc((size_t)n * sizeof(float));
        float* col = xmalloc((size_t)rows * sizeof(float));
        ora_rht(x, dtype, rows, cols, signs, 0, b);
        ora_rht(b, 0, rows, cols, signs, 1, a);
        ora_rht_column(x, dtype, rows, cols, cols - 1, signs, col);
        for (int64_t i = 0; i < rows; ++i)
            expect(col[i] == b[i * cols + cols - 1], "rht column equals the whole transform");
        free(b);
        free(a);
        free(col);
    }
    free(y);
}

static void gemms(int64_t m, int64_t n, int64_t k)
{
    uint8_t* ac = xmalloc((size_t)(m * k / 2));
    uint8_t* bc = xmalloc((size_t)(n * k / 2));
    uint8_t* as = xmalloc((size_t)(m * k / 16));
    uint8_t* bs = xmalloc((size_t)(n * k / 16));
    for (int64_t i = 0; i < m * k / 2; ++i) ac[i] = (uint8_t)next_u32();
    for (int64_t i = 0; i < n * k / 2; ++i) bc[i] = (uint8_t)next_u32();
    for (int64_t i = 0; i < m * k / 16; ++i) as[i] = (uint8_t)(118 + next_u32() % 16);
    for (int64_t i = 0; i < n * k / 16; ++i) bs[i] = (uint8_t)(118 + next_u32() % 16);
    double* c = xmalloc((size_t)(m * n) * sizeof(double));
    double* cabs = xmalloc((size_t)(m * n) * sizeof(double));
    ora_gemm_mxfp4(ac, as, bc, bs, m, n, k, c, cabs);   /* reads the first k/32 scales per row */
    ora_gemm_mxfp4(ac, as, bc, bs, m, n, k, c, NULL);
    ora_gemm_nvfp4(ac, as, 0.75f, bc, bs, 3.0f, m, n, k, 0, c, cabs);
    ora_gemm_nvfp4(ac, as, 0.75f, bc, bs, 3.0f, m, n, k, 12, c, cabs);   /* IF4 x IF4: flagged scales */
    ora_gemm_nvfp4(ac, as, 0.75f, bc, bs, 3.0f, m, n, k, 4, c, NULL);
    if (m % 16 == 0 && n % 16 == 0) {
        /* 16x16 tiles: exact-size tile arrays, so a read past [rows/16][k/16] is caught */
        uint8_t* ta = xmalloc((size_t)(m / 16 * (k / 16)));
        uint8_t* tb = xmalloc((size_t)(n / 16 * (k / 16)));
        memcpy(ta, as, (size_t)(m / 16 * (k / 16)));
        memcpy(tb, bs, (size_t)(n / 16 * (k / 16)));
        ora_gemm_nvfp4(ac, ta, 0.75f, bc, tb, 3.0f, m, n, k, 3, c, cabs);
        ora_gemm_nvfp4(ac, ta, 0.75f, bc, bs, 3.0f, m, n, k, 1, c, cabs);
        ora_gemm_nvfp4(ac, as, 0.75f, bc, tb, 3.0f, m, n, k, 2, c, NULL);
        free(ta);
        free(tb);
    }
    free(ac);
    free(bc);
    free(as);
    free(bs);
    free(c);
    free(cabs);
}

int main(void)
{
    /* element and scale codecs over their whole domains */
    for (int c = 0; c < 16; ++c) {
        expect(ora_e2m1_rtn(ora_e2m1_decode((uint8_t)c)) == (c == 8 ? 8 : c), "e2m1 round trip");
        (void)ora_int4_decode((uint8_t)c);
        (void)ora_e2m1_sr(ora_e2m1_decode((uint8_t)c), next_u32());
    }
    for (int c = 0; c < 256; ++c) {
        (void)ora_e4m3_decode((uint8_t)c);
        (void)ora_e8m0_decode((uint8_t)c);
    }
    for (int c = 0; c < 64; ++c) {
        (void)ora_fp6_decode(0, (uint8_t)c);
        (void)ora_fp6_decode(1, (uint8_t)c);
    }
    const float probes[] = {0.0f, -0.0f, 1e-45f, 1e-38f, 0.25f, 0.75f, 2.5f, 5.0f, 6.0f, 447.9f, 448.0f,
                            464.0f, 1e30f, 3.4e38f, -3.4e38f};
    for (size_t i = 0; i < sizeof(probes) / sizeof(probes[0]); ++i) {
        const float v = probes[i];
        (void)ora_e2m1_rtn(v);
        (void)ora_e2m1_sr(v, 0xFFFFu);
        (void)ora_e4m3_encode(fabsf(v));
        (void)ora_e8m0_encode(fabsf(v));
        (void)ora_fp6_rtn(0, v);
        (void)ora_fp6_rtn(1, v);
        (void)ora_tensor_scale(fabsf(v));
    }
    {
        const int64_t n = 257;
        float* v = make_f32(n, 3.0f, 0);
        uint32_t* r = xmalloc((size_t)n * sizeof(uint32_t));
        uint64_t* idx = xmalloc((size_t)n * sizeof(uint64_t));
        uint8_t* out = xmalloc((size_t)n);
        for (int64_t i = 0; i < n; ++i) {
            r[i] = next_u32() & 0xFFFFu;
            idx[i] = ((uint64_t)next_u32() << 20) ^ (uint64_t)i;
            v[i] = fabsf(v[i]) * ((i & 1) ? 1.0f : -1.0f);
        }
        ora_e2m1_rtn_array(v, n, out);
        ora_e2m1_sr_array(v, r, n, out);
        for (int64_t i = 0; i < n; ++i) v[i] = fabsf(v[i]) * 40.0f;
        ora_e4m3_encode_array(v, n, out);
        ora_e8m0_encode_array(v, n, out);
        ora_sr_bits16_array(12345u, 1u, idx, n, r);
        for (int64_t i = 0; i < n; ++i) expect(r[i] == ora_sr_bits16(12345u, 1u, idx[i]), "sr bits array");
        free(v);
        free(r);
        free(idx);
        free(out);
    }
    {
        uint32_t ctr[4] = {1u, 2u, 3u, 4u}, key[2] = {5u, 6u}, out[4];
        ora_philox4x32_10(ctr, key, out);
        for (int i = 0; i < 128; ++i)
            for (int t = 0; t < 128; t += 17) (void)ora_hadamard_entry(i, t);
    }
    {
        float* x = make_f32(4096, 1.0f, 0);
        float* y = xmalloc(4096 * sizeof(float));
        ora_plain_block_roundtrip(x, 4096, 4096, y);
        ora_plain_block_roundtrip(x, 4096, 32, y);
        ora_plain_block_roundtrip(x, 4096, 16, y);
        free(x);
        free(y);
    }

    /* the quantizers: several shapes and value kinds, fp32 and bf16 */
    const int64_t shapes[][2] = {{1, 16}, {1, 32}, {16, 16}, {16, 8}, {3, 96}, {37, 48}, {128, 40}, {256, 64}};
    for (size_t si = 0; si < sizeof(shapes) / sizeof(shapes[0]); ++si) {
        const int64_t rows = shapes[si][0], cols = shapes[si][1];
        for (int kind = 0; kind < 5; ++kind) {
            float* x = make_f32(rows * cols, kind == 0 ? 2.0f : 1.0f, kind);
            uint16_t* xb = to_bf16(x, rows * cols);
            quantizers(x, ORA_F32, rows, cols);
            quantizers(xb, ORA_BF16, rows, cols);
            free(x);
            free(xb);
        }
    }
    gemms(3, 5, 128);
    gemms(1, 1, 256);
    gemms(32, 48, 128);

    if (failures) {
        fprintf(stderr, "%d failures\n", failures);
        return 1;
    }
    printf("oracle driver: every oracle entry point ran clean\n");
    return 0;
}
