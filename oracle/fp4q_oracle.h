/*
 * fp4q_oracle.h -- declarations of the CPU oracle (test infrastructure only).
 * See fp4q_oracle.c for the definitions and the passages each one follows.
 * This header is private to oracle/: the HIP library never includes it.
 */
#ifndef FP4Q_ORACLE_H
#define FP4Q_ORACLE_H

#include <stdint.h>

#define ORA_F32 0
#define ORA_BF16 1
#define ORA_RTN 0
#define ORA_SR 1

void ora_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]);
uint32_t ora_sr_bits16(uint64_t seed, uint32_t stream, uint64_t idx);
void ora_rht_signs(uint64_t seed, uint32_t signs[4]);

float ora_e2m1_decode(uint8_t nibble);
uint8_t ora_e2m1_rtn(float v);
uint8_t ora_e2m1_sr(float v, uint32_t r16);
float ora_e4m3_decode(uint8_t code);
uint8_t ora_e4m3_encode(float y);
float ora_e8m0_decode(uint8_t code);
uint8_t ora_e8m0_encode(float y);
float ora_int4_decode(uint8_t nibble);

float ora_amax(const void* x, int dtype, int64_t n);
float ora_tensor_scale(float amax);

void ora_quantize_nvfp4_strided(const void* x, int dtype, int64_t lrows, int64_t lcols,
                                int64_t sr, int64_t sc, float gs, int rnd, uint64_t seed,
                                uint32_t stream, int64_t row0, uint8_t* codes, uint8_t* scales);
void ora_quantize_nvfp4(const void* x, int dtype, int64_t rows, int64_t cols, int colwise,
                        float gs, int rnd, uint64_t seed, uint8_t* codes, uint8_t* scales);
void ora_quantize_nvfp4_2d(const void* x, int dtype, int64_t rows, int64_t cols, float gs,
                           uint8_t* codes, uint8_t* scales);
void ora_quantize_mxfp4(const void* x, int dtype, int64_t rows, int64_t cols, int rnd,
                        uint64_t seed, uint8_t* codes, uint8_t* scales);
void ora_quantize_if4(const void* x, int dtype, int64_t rows, int64_t cols, float gs,
                      uint8_t* codes, uint8_t* scales);
void ora_dequantize(int fmt, const uint8_t* codes, const uint8_t* scales, float gs,
                    int64_t rows, int64_t cols, float* y);

void ora_gemm_mxfp4(const uint8_t* a_codes, const uint8_t* a_scales, const uint8_t* b_codes,
                    const uint8_t* b_scales, int64_t m, int64_t n, int64_t k, double* c, double* cabs);
/* flags: bit 0 / 1 A / B has 16x16 scale tiles; bit 2 / 3 A / B is IF4. */
void ora_gemm_nvfp4(const uint8_t* a_codes, const uint8_t* a_scales, float gs_a, const uint8_t* b_codes,
                    const uint8_t* b_scales, float gs_b, int64_t m, int64_t n, int64_t k, int flags,
                    double* c, double* cabs);
float ora_fp6_decode(int fmt, uint8_t code);
uint8_t ora_fp6_rtn(int fmt, float v);
void ora_quantize_mxfp6(const void* x, int dtype, int64_t rows, int64_t cols, int fmt, uint8_t* codes,
                        uint8_t* scales);
void ora_dequantize_mxfp6(int fmt, const uint8_t* codes, const uint8_t* scales, int64_t rows, int64_t cols,
                          float* y);
int ora_hadamard_entry(int i, int t);
void ora_rht(const void* x, int dtype, int64_t rows, int64_t cols, const uint32_t signs[4],
             int inverse, float* y);
void ora_rht_column(const void* x, int dtype, int64_t rows, int64_t cols, int64_t j,
                    const uint32_t signs[4], float* y);

void ora_plain_block_roundtrip(const float* x, int64_t n, int64_t block, float* y);

#define ORA_VAR_46 0
#define ORA_VAR_NVINT4 1
#define ORA_VAR_IF3 2
#define ORA_VAR_IF4 3
#define ORA_VAR_IF6 4
float ora_fp3_decode(uint8_t code);
uint8_t ora_fp3_rtn(float v);
int64_t ora_variant_row_bytes(int var, int64_t cols);
float ora_variant_tensor_scale(int var, float amax);
void ora_quantize_variant(const void* x, int dtype, int64_t rows, int64_t cols, int var, float gs,
                          uint8_t* codes, uint8_t* scales);
void ora_dequantize_variant(int var, const uint8_t* codes, const uint8_t* scales, float gs, int64_t rows,
                            int64_t cols, float* y);



void ora_e2m1_rtn_array(const float* v, int64_t n, uint8_t* out);
void ora_e2m1_sr_array(const float* v, const uint32_t* r16, int64_t n, uint8_t* out);
void ora_e4m3_encode_array(const float* y, int64_t n, uint8_t* out);
void ora_e8m0_encode_array(const float* y, int64_t n, uint8_t* out);
void ora_sr_bits16_array(uint64_t seed, uint32_t stream, const uint64_t* idx, int64_t n, uint32_t* out);
#endif
