/*
 * fp4q.h -- C ABI of libfp4q: block-scaled FP4 quantization on MI355X (gfx950).
 *
 * Sources of the operations (page, then section):
 *  [NV] qiita.com/nishiha/items/b98c2b931d588c4c81d5 (notes on NVIDIA's NVFP4
 *       pretraining recipe): "NVFP4データの変換" (E2M1), "Blockwise" (1x16 blocks),
 *       "誤差逆伝播と転置" (backprop needs the transposed operands), "NVFP4フロー図"
 *       (the forward, data- and weight-gradient GEMMs on quantized operands), "2D scaling",
 *       "ランダムアダマール変換" (RHT), "確率的丸め" (stochastic rounding),
 *       "NVFP4の表現できる最大値", "scaleの導出" (tensor and block scales).
 *  [GL] ultralytics.com/ja/glossary/fp4 (glossary "FP4"): "FP4の仕組み"
 *       (MXFP4: 32 values + E8M0 scale; NVFP4: 16 values + E4M3 scale + FP32 scale),
 *       "FP4による推論と学習" (FP4 products accumulated in higher precision),
 *       "FP4モデルのデプロイ" (MXFP4 native on the MI350 family).
 *  [IF] gist.science/ja/paper/2603.28765 (explainer of "Adaptive Block-Scaled Data
 *       Types"): "2. 提案手法：IF4" (FP4/INT4 per block, sign-bit flag, 6/7 rule).
 *  [F6] blog.ast.moe/blog/2026-09-24 ("FP6から考えるLLM量子化"):
 *       "FP6で隣り合う値の間隔を見てみる" (E8M0 scale with round-to-nearest-even).
 *
 * Conventions for every call:
 *  - Tensor pointers are HIP DEVICE pointers to dense row-major matrices (row stride
 *    == cols).  `rows` x `cols` is the shape of the input matrix.
 *  - Tensor, code and scale pointers must be 16-byte aligned, the float[1] amax and
 *    tensor_scale pointers 4-byte aligned (FP4Q_E_ALIGN otherwise).
 *  - Inputs and outputs must not overlap.  The caller allocates every buffer and
 *    keeps it alive until the work on `stream` has completed.  No call allocates or
 *    frees memory, synchronizes, or keeps state between calls, except through an
 *    fp4q_workspace the caller creates once and passes in (below).
 *  - A call validates its arguments on the host, enqueues its kernels on `stream`
 *    (0 = the null stream) and returns without synchronizing.  On any validation
 *    error nothing is enqueued.  Device faults surface at the caller's next sync.
 *  - Inputs must be finite; codes for non-finite inputs are unspecified.
 *  - All calls are reentrant; calls on different streams may run concurrently
 *    when their output buffers, and their workspaces, are distinct.
 *  - The quantize, transform, dequantize and GEMM calls are safe to capture into a
 *    HIP graph (they enqueue kernels only: no memset, allocation or host
 *    synchronization); a captured call gives correct results on every replay, also
 *    when the inputs change between replays.
 *
 * Packed layouts (all byte arrays):
 *  - codes: element 2k of a logical row in bits 0-3 of byte k, element 2k+1 in
 *    bits 4-7.  E2M1 nibble = sign(1) exp(2) man(1); IF4 INT4 nibble = two's
 *    complement in -7..7.
 *  - E4M3 scale byte: OCP e4m3fn, never negative; IF4 sets bit 7 for INT4 blocks.
 *  - E8M0 scale byte: value 2^(byte-127), 0..254.
 */
#ifndef FP4Q_H
#define FP4Q_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FP4Q_ABI_VERSION 10

typedef enum {
    FP4Q_OK = 0,
    FP4Q_E_NULL = 1,   /* a required pointer is NULL */
    FP4Q_E_SHAPE = 2,  /* rows/cols <= 0 or not a multiple of the block (see each call) */
    FP4Q_E_ALIGN = 3,  /* a device pointer is not 16-byte aligned */
    FP4Q_E_ARG = 4,    /* invalid enum, empty layout mask, or an unsupported combination */
    FP4Q_E_HIP = 5     /* the HIP runtime reported an error while enqueueing */
} fp4q_status;

typedef enum { FP4Q_F32 = 0, FP4Q_BF16 = 1 } fp4q_dtype;
typedef enum { FP4Q_RTN = 0, FP4Q_SR = 1 } fp4q_round;
typedef enum {
    FP4Q_FMT_NVFP4 = 0, FP4Q_FMT_NVFP4_2D = 1, FP4Q_FMT_MXFP4 = 2, FP4Q_FMT_IF4 = 3,
    FP4Q_FMT_MXFP6_E2M3 = 4, FP4Q_FMT_MXFP6_E3M2 = 5
} fp4q_format;
typedef enum { FP4Q_FP6_E2M3 = 0, FP4Q_FP6_E3M2 = 1 } fp4q_fp6;

#define FP4Q_ROWWISE 1u
#define FP4Q_COLWISE 2u

/* amax_mode: COMPUTE = the call writes max|x| to *amax; GIVEN = *amax is read as the
 * tensor's max magnitude (e.g. produced upstream) and not recomputed. */
#define FP4Q_AMAX_COMPUTE 0u
#define FP4Q_AMAX_GIVEN 1u

/*
 * Workspace: a small piece of device memory (FP4Q_WORKSPACE_BYTES) through which the
 * workgroups of a call that computes a tensor amax exchange partial maxima
 * [NV "scaleの導出": the tensor scale needs the maximum of the whole tensor before any
 * element is encoded].  With a workspace,
 *   - fp4q_quantize_nvfp4 (AMAX_COMPUTE, no RHT) finds the amax and quantizes in ONE
 *     read of x when the tensor fits one co-resident grid (about 64 MB of bf16);
 *   - two-pass calls (an amax pass, then the quantizer) hand the amax over in the
 *     workspace instead of zeroing the caller's float first (one launch fewer);
 *   - fp4q_quantize_mxfp4 can report the tensor amax from its own read of x.
 * Passing NULL instead is always valid: the calls then zero *amax with a one-thread
 * kernel and post into it (MXFP4's amax report needs a workspace: FP4Q_E_NULL).
 *
 * Ownership and rules: fp4q_workspace_create allocates and clears the memory on the
 * CURRENT device and synchronizes the device before it returns; it is the only call
 * that allocates.  fp4q_workspace_destroy frees it (the caller first ensures that no
 * enqueued work still uses it).  A workspace belongs to the device it was created on
 * (FP4Q_E_ARG on another device) and must not be used by two calls that may run at the
 * same time (e.g. on two streams without an order between them): its words are the
 * calls' shared state.  It is not thread-safe.  After a call returns FP4Q_E_HIP its
 * contents are undefined: destroy and re-create it.  Under stream capture the
 * one-pass kernel is not used (its launch number lives on the host and would repeat
 * on every replay); the two-pass protocol keeps all of its state on the device.
 */
typedef struct fp4q_workspace fp4q_workspace;
#define FP4Q_WORKSPACE_BYTES 36864

fp4q_status fp4q_workspace_create(fp4q_workspace** ws);
fp4q_status fp4q_workspace_destroy(fp4q_workspace* ws);

/* One-pass kernel: a workgroup whose wait for another workgroup's partial maximum
 * exceeds this limit reads the corresponding part of x itself, so results never depend
 * on every workgroup being resident.  On an idle GPU the grid is resident and no wait
 * runs out.  When another kernel occupies the GPU at the same time (e.g. a concurrent
 * stream), waits can run out and each such call costs about this limit more (still
 * exact); lower it, or pass AMAX_GIVEN, where that matters.  Default 200 us; 0 makes
 * every wait give up at once (slow, but exact).  Applies to calls enqueued afterwards. */
fp4q_status fp4q_workspace_set_wait(fp4q_workspace* ws, uint32_t microseconds);

/* Waits for `stream`, then stores in *count how many waits of one-pass calls on this
 * workspace ran out and were answered by reading x (0 when the grid was resident). */
fp4q_status fp4q_workspace_fallbacks(fp4q_workspace* ws, hipStream_t stream, uint32_t* count);

/*
 * NVFP4 with 1x16 blocks [NV "scaleの導出", "Blockwise", "誤差逆伝播と転置"; GL].
 * Tensor scale gs = 2688 / amax (amax = 0 -> 1; overflow -> FLT_MAX), written to
 * *tensor_scale.  Per 16-element block: s = E4M3(fl(fl(bamax * gs) / 6)); each element
 * v = fl(fl(x * gs) / s) rounded onto E2M1 (RTN: nearest, ties to even code,
 * saturating; SR: up iff frac + u >= 1 with a 16-bit Philox4x32-10 draw u keyed on
 * (sr_seed, element index), [NV "確率的丸め"]).  A block whose scale is 0 gives
 * signed zeros.
 *   layouts   FP4Q_ROWWISE: blocks along rows;   row_codes [rows][cols/2], row_scales [rows][cols/16]
 *             FP4Q_COLWISE: quantization of X^T; col_codes [cols][rows/2], col_scales [cols][rows/16]
 *             Both bits may be set; both use the same gs.
 *   rht_signs HOST pointer to 4 words (bit t of word t/32 set means sign -1) or NULL.
 *             Non-NULL applies the 128x128 random Hadamard transform along rows in
 *             chunks of 128 before quantizing [NV "ランダムアダマール変換"]; requires
 *             layouts == FP4Q_COLWISE, rows % 128 == 0 and cols < 2^27.  The amax and
 *             gs are then those of the transformed matrix, and the quantized values are
 *             exactly those fp4q_rht returns for the same x and dt: for bf16 the
 *             contraction runs on MFMA, for fp32 as 7 butterfly stages of fp32 adds.
 *   amax, tensor_scale  device float[1] each.
 *   ws        workspace or NULL (see above).
 * Shapes: ROWWISE needs cols % 16 == 0; COLWISE needs rows % 16 == 0 and cols % 8 == 0.
 * SR uses stream 0 for the row-wise output and stream 1 for the column-wise output;
 * element index idx = row * lcols + col of the logical (output) matrix.  One
 * Philox4x32-10 call, counter {lo32(idx/8), hi32(idx/8), stream, 0} and key
 * {lo32(sr_seed), hi32(sr_seed)}, serves the 8 elements idx/8*8 .. +7: element idx
 * takes the high 16 bits of output word (idx/2) % 4 when idx is even, the low 16 bits
 * when idx is odd, as u = draw / 2^16 (MXFP4 uses the same layout with stream 0).
 */
fp4q_status fp4q_quantize_nvfp4(const void* x, fp4q_dtype dt, int64_t rows, int64_t cols,
                                unsigned layouts, fp4q_round rnd, uint64_t sr_seed,
                                const uint32_t* rht_signs, unsigned amax_mode, float* amax,
                                float* tensor_scale, uint8_t* row_codes, uint8_t* row_scales,
                                uint8_t* col_codes, uint8_t* col_scales, fp4q_workspace* ws,
                                hipStream_t stream);

/*
 * fp4q_quantize_nvfp4 for callers that cannot allocate (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc): the same arguments, checks and
 * results as fp4q_quantize_nvfp4, without a workspace argument.  Its workspace is a
 * file-scope device array of FP4Q_WORKSPACE_BYTES (36 KiB) inside the library, one copy
 * per GPU, held from the first call on that GPU until the process ends; the first call
 * on a GPU looks up the array's address and clears it with a kernel on `stream`.  The
 * array's size does not depend on the input, so every shape fp4q_quantize_nvfp4 accepts
 * is accepted.  The call allocates nothing (no hipMalloc, no hipFree).  All calls on one
 * GPU share the array: calls that may overlap on one GPU (e.g. on two streams without an
 * order between them) race; order them, or use fp4q_quantize_nvfp4 with one workspace
 * per stream.  The host part of a call is serialized by a lock.
 */
fp4q_status fp4q_quantize_nvfp4_noalloc(const void* x, fp4q_dtype dt, int64_t rows, int64_t cols,
                                        unsigned layouts, fp4q_round rnd, uint64_t sr_seed,
                                        const uint32_t* rht_signs, unsigned amax_mode, float* amax,
                                        float* tensor_scale, uint8_t* row_codes, uint8_t* row_scales,
                                        uint8_t* col_codes, uint8_t* col_scales, hipStream_t stream);

/*
 * NVFP4 with 16x16 blocks for weights [NV "2D scaling"]: one E4M3 scale per 16x16
 * tile, so quantizing W^T gives exactly the transposed codes and scales.  RTN only.
 *   codes [rows][cols/2], scales [rows/16][cols/16];
 *   codes_t optional (NULL to skip): [cols][rows/2], the same codes in the layout of
 *   W^T, i.e. the codes of q(W^T).
 *   ws      workspace or NULL.
 * Shapes: rows % 16 == 0, cols % 16 == 0.
 */
fp4q_status fp4q_quantize_nvfp4_2d(const void* x, fp4q_dtype dt, int64_t rows, int64_t cols,
                                   unsigned amax_mode, float* amax, float* tensor_scale,
                                   uint8_t* codes, uint8_t* scales, uint8_t* codes_t,
                                   fp4q_workspace* ws, hipStream_t stream);

/*
 * MXFP4: 32 elements + one E8M0 scale [GL "FP4の仕組み"; F6].  Per block the scale
 * code is E8M0_RNE(fl(bamax / 6)) (nearest power of two, ties at significand 1.5 to
 * the even code); elements are x * 2^(127 - code) rounded onto E2M1 (RTN or SR as
 * above, stream 0).  No tensor scale.
 *   codes [rows][cols/2], scales [rows][cols/32].   Shapes: cols % 32 == 0.
 *   amax  device float[1] or NULL.  Non-NULL also writes max|x| over the tensor, the
 *         value fp4q_amax returns, from the same read of x: a caller that quantizes
 *         one tensor to MXFP4 and to an amax-scaled format passes it on with
 *         FP4Q_AMAX_GIVEN instead of running an amax pass.  Needs a workspace
 *         (FP4Q_E_NULL if ws is NULL).
 */
fp4q_status fp4q_quantize_mxfp4(const void* x, fp4q_dtype dt, int64_t rows, int64_t cols,
                                fp4q_round rnd, uint64_t sr_seed, uint8_t* codes, uint8_t* scales,
                                float* amax, fp4q_workspace* ws, hipStream_t stream);

/*
 * MX FP6 [F6 "FP6で隣り合う値の間隔を見てみる", "量子化と6bitの保存"]: the OCP MX six-bit
 * element formats E2M3 (bias 1, largest 7.5) and E3M2 (bias 3, largest 28, smallest
 * step 0.0625), subnormals at exponent 0, no Inf or NaN; blocks of 32 with an E8M0
 * scale chosen as for MXFP4 with the format's largest value in place of 6:
 * E8M0_RNE(fl(bamax / max)).  Elements x * 2^(127 - code) round to the nearest code,
 * ties to the even code, saturating at the largest; the sign bit is copied.  Four codes
 * per three bytes: code j of a group of four in bits 6j .. 6j+5 of the little-endian
 * 24-bit word the three bytes form.  RTN only.
 *   codes [rows][3*cols/4], E8M0 scales [rows][cols/32].   Shapes: cols % 32 == 0.
 * fp4q_dequantize with FP4Q_FMT_MXFP6_E2M3 / _E3M2 decodes it (tensor_scale unused).
 */
fp4q_status fp4q_quantize_mxfp6(const void* x, fp4q_dtype dt, int64_t rows, int64_t cols, fp4q_fp6 fmt,
                                uint8_t* codes, uint8_t* scales, hipStream_t stream);

/*
 * IF4 [IF "2. 提案手法：IF4"]: NVFP4 1x16 row-wise scaling, then per block the
 * FP4 candidate and the INT4 candidate q = clamp(rint(fl(v * fl(7/6))), -7, 7)
 * (restored as fl(q * fl(6/7))) are compared by sum_i fma-accumulated (v_i - r_i)^2,
 * i ascending; INT4 is kept only if strictly lower and flagged in bit 7 of the
 * block's E4M3 scale byte.  RTN only.
 *   codes [rows][cols/2], scales [rows][cols/16].   Shapes: cols % 16 == 0.
 *   ws    workspace or NULL.
 */
fp4q_status fp4q_quantize_if4(const void* x, fp4q_dtype dt, int64_t rows, int64_t cols,
                              unsigned amax_mode, float* amax, float* tensor_scale,
                              uint8_t* codes, uint8_t* scales, fp4q_workspace* ws,
                              hipStream_t stream);

/*
 * Block-format variants on NVFP4's two-level scaling, the formats IF4 is compared with
 * and its extensions [IF "1. 背景と問題点", "2. 提案手法：IF4", "3. 主要な貢献"]:
 *   FP4Q_VAR_46      Four Over Six: E2M1 with the block maximum mapped to 4 instead of 6
 *                    (+-6 are never produced); same code and scale layout as NVFP4.
 *   FP4Q_VAR_NVINT4  INT4 elements q = clamp(rint(v), -7, 7), block maximum 7.
 *   FP4Q_VAR_IF3     per block FP3 E2M0 (0, 1, 2, 4) or INT3 q = clamp(rint(fl(v * fl(3/4))),
 *                    -3, 3) restored as fl(q * fl(4/3)); block maximum 4.
 *   FP4Q_VAR_IF4     IF4 as fp4q_quantize_if4 writes it (the same bytes).
 *   FP4Q_VAR_IF6     per block FP6 E2M3 (max 7.5) or INT6 with fl(31/7.5), restored with
 *                    fl(7.5/31); block maximum 7.5.
 * For each, with M the block maximum: gs = 448 * M / amax (amax = 0 -> 1; overflow ->
 * FLT_MAX), written to *tensor_scale; per 16-element row block s = E4M3(fl(fl(bamax * gs)
 * / M)); v = fl(fl(x * gs) / s); the IF variants keep the candidate with the smaller
 * fma-accumulated squared error (INT only if strictly smaller) and set bit 7 of the scale
 * byte for INT.  INT codes are two's complement; FP codes sign-magnitude.
 *   codes  [rows][cols * bits / 8] with bits = 4 (46, NVINT4, IF4), 3 (IF3) or 6 (IF6):
 *          4-bit codes two per byte (element 2k low nibble); 3-bit codes eight per three
 *          bytes and 6-bit codes four per three bytes, code j of a group at bits
 *          bits*j.. of the little-endian 24-bit word.
 *   scales [rows][cols/16], E4M3 (+ flag).   Shapes: cols % 16 == 0.   RTN only.
 *   ws     workspace or NULL (as fp4q_quantize_if4).
 */
typedef enum {
    FP4Q_VAR_46 = 0, FP4Q_VAR_NVINT4 = 1, FP4Q_VAR_IF3 = 2, FP4Q_VAR_IF4 = 3, FP4Q_VAR_IF6 = 4
} fp4q_variant;

fp4q_status fp4q_quantize_variant(const void* x, fp4q_dtype dt, int64_t rows, int64_t cols, fp4q_variant var,
                                  unsigned amax_mode, float* amax, float* tensor_scale, uint8_t* codes,
                                  uint8_t* scales, fp4q_workspace* ws, hipStream_t stream);

/* Dequantizes a variant: x_hat = fl(fl(r * s) / gs), r the FP value, or the INT restore
 * (q for NVINT4, fl(q * cinv) for flagged IF blocks); gs = *tensor_scale (device float).
 * out_dt FP4Q_F32 or FP4Q_BF16 (RNE of the fp32 result).  Layouts as above. */
fp4q_status fp4q_dequantize_variant(fp4q_variant var, const uint8_t* codes, const uint8_t* scales,
                                    const float* tensor_scale, int64_t rows, int64_t cols, fp4q_dtype out_dt,
                                    void* y, hipStream_t stream);

/*
 * Random Hadamard transform along rows [NV "ランダムアダマール変換"], per chunk of
 * 128 rows, R = S H / sqrt(128) with Sylvester H and S = diag(signs):
 *   inverse == 0:  y = R^T x    (y[128c+i][j] = sum_t H[i][t] s_t x[128c+t][j] / sqrt(128))
 *   inverse != 0:  y = R x      (undoes the forward transform)
 * dt == FP4Q_BF16: contraction on MFMA (bf16 operands, fp32 accumulation);
 * dt == FP4Q_F32: fast Walsh-Hadamard butterflies in fp32 (7 rounded adds per output).
 * The forward transform is the one fp4q_quantize_nvfp4 applies for the same dt, bit
 * for bit.
 *   signs  HOST pointer to 4 words.   y  device float [rows][cols].
 * Shapes: rows % 128 == 0, cols % 8 == 0.
 */
fp4q_status fp4q_rht(const void* x, fp4q_dtype dt, int64_t rows, int64_t cols,
                     const uint32_t* signs, int inverse, float* y, hipStream_t stream);

/*
 * FP4 GEMM consumer [NV "NVFP4フロー図"; GL "FP4による推論と学習"]: the product that
 * follows quantization, on two operands quantized along the reduction dimension k:
 *   c[i][j] = sum_t a(i,t) * b(j,t),   a(i,t) = E2M1 * 2^(a_scale - 127), likewise b,
 * i.e. C = A B^T with A [m][k] and B [n][k] both row-wise MXFP4 as fp4q_quantize_mxfp4
 * writes them (codes [rows][k/2], E8M0 scales [rows][k/32]).  For Y = X W^T pass the
 * activation X as A and the weight W as B.  Products and sums run on the block-scaled
 * MFMA with fp32 accumulation; the summation order is the hardware's.
 *   out_dt FP4Q_F32: c is float [m][n];  FP4Q_BF16: bf16 [m][n] = RNE(fp32 result).
 * Shapes: m >= 1, n >= 1, k >= 128 with k % 128 == 0 and k <= 2^25, m, n < 2^31.
 *   amax   optional device float (NULL: not computed), 4-byte aligned: receives
 *          max |c[i][j]| over the m x n outputs as stored (after the bf16 rounding for
 *          FP4Q_BF16), i.e. the tensor amax that an NVFP4 or IF4 quantization of C
 *          needs [NV "scaleの導出"], produced by the GEMM's own epilogue so that C is
 *          not read again for it; pass it on with FP4Q_AMAX_GIVEN.  It is set to 0 on
 *          the stream before the GEMM starts; a NaN output makes it a NaN.
 */
fp4q_status fp4q_gemm_mxfp4(const uint8_t* a_codes, const uint8_t* a_scales,
                            const uint8_t* b_codes, const uint8_t* b_scales,
                            int64_t m, int64_t n, int64_t k, fp4q_dtype out_dt, void* c,
                            float* amax, hipStream_t stream);

/*
 * The same product over two row-wise NVFP4 1x16 operands [NV "NVFP4フロー図";
 * NV "scaleの導出"], whose dequantized values are r * s / gs:
 *   c[i][j] = (sum_t (r_a s_a)(r_b s_b)) / (gs_a gs_b),
 * with codes [rows][k/2], E4M3 scales [rows][k/16] as fp4q_quantize_nvfp4 writes them
 * (row-wise, or the column-wise output of the transposed operand, e.g. the Wgrad pair
 * after the RHT), and gs_a = *a_tensor_scale, gs_b = *b_tensor_scale (device floats,
 * the encode scales the quantizer stored).  Each r * s (at most six significant bits)
 * is decoded exactly to f16 (bf16 where an IF4 operand takes part, see below) and
 * multiplied on the 16-bit MFMA with fp32 accumulation; the sums are multiplied by
 * fl(1 / fl(gs_a gs_b)).
 *   out_dt FP4Q_F32: float [m][n];  FP4Q_BF16: bf16 [m][n] = RNE(fp32 result).
 *   operand_flags  0 or an OR of:
 *     FP4Q_TILES_A / FP4Q_TILES_B: that operand carries NVFP4 16x16 scales as
 *          fp4q_quantize_nvfp4_2d writes them [NV "2D scaling"], one E4M3 byte per
 *          16x16 tile, [rows/16][k/16] (rows % 16 == 0), e.g. the weight W as B in
 *          Y = X W^T.  For W^T (the data-gradient product) pass codes_t and the
 *          transposed tile array: quantizing W^T gives exactly those codes and scales.
 *     FP4Q_IF4_A / FP4Q_IF4_B: that operand is IF4 as fp4q_quantize_if4 writes it
 *          [IF "2. 提案手法：IF4"]: a scale byte with bit 7 set marks an INT4 block whose
 *          element is fl(q * fl(6/7)) * s (q the two's-complement nibble, s the E4M3 value
 *          of the low seven bits).  Such an element e has up to 24 significant bits; the
 *          MFMA takes it as hi + lo, hi = bf16(e) and lo = bf16(e - hi), with a second
 *          MFMA for the lo parts (twice the MFMA work for one IF4 operand, three times for
 *          two): hi + lo is within (2^-16 + 2^-24) |e| of the exact element (bf16
 *          rounding twice, after the fp32 rounding of e), so one IF4 operand puts each
 *          product within that of the exact one; with both IF4 the lo x lo product (at
 *          most about 2^-16 of the product) is left out, about 3 * 2^-16 in all.
 *     TILES and IF4 on the same operand: FP4Q_E_ARG (IF4 blocks are 1x16).
 * Shapes and amax as fp4q_gemm_mxfp4.
 */
#define FP4Q_TILES_A 1u
#define FP4Q_TILES_B 2u
#define FP4Q_IF4_A 4u
#define FP4Q_IF4_B 8u
fp4q_status fp4q_gemm_nvfp4(const uint8_t* a_codes, const uint8_t* a_scales, const float* a_tensor_scale,
                            const uint8_t* b_codes, const uint8_t* b_scales, const float* b_tensor_scale,
                            int64_t m, int64_t n, int64_t k, unsigned operand_flags, fp4q_dtype out_dt, void* c,
                            float* amax, hipStream_t stream);

/*
 * Dequantize packed codes back to values.  rows x cols is the LOGICAL shape of the
 * quantized matrix (for a column-wise NVFP4 output pass (cols_in, rows_in)).
 *   NVFP4, NVFP4_2D, IF4: x_hat = fl(fl(r * s) / gs), r = the E2M1 value, or for an
 *     IF4 block flagged INT4 r = fl(q * fl(6/7)); gs = *tensor_scale (device float).
 *   MXFP4: x_hat = r * 2^(code-127); tensor_scale may be NULL.
 *   MXFP6_E2M3 / _E3M2: x_hat = fp6(code) * 2^(scale-127), codes [rows][3*cols/4];
 *     tensor_scale unused.
 *   out_dt FP4Q_F32 writes float; FP4Q_BF16 writes bf16 = RNE(float result).
 * Shapes as for the matching quantize call.
 */
fp4q_status fp4q_dequantize(fp4q_format fmt, const uint8_t* codes, const uint8_t* scales,
                            const float* tensor_scale, int64_t rows, int64_t cols,
                            fp4q_dtype out_dt, void* y, hipStream_t stream);

/* max |x| over the whole matrix, written to device float *amax. */
fp4q_status fp4q_amax(const void* x, fp4q_dtype dt, int64_t rows, int64_t cols, float* amax,
                      hipStream_t stream);

/* The RHT sign mask for a seed: one Philox4x32-10 call with counter {0,0,0,1} and key
 * {lo32(seed), hi32(seed)}; its 128 output bits are the signs (host only). */
void fp4q_rht_signs_from_seed(uint64_t seed, uint32_t signs[4]);

const char* fp4q_status_string(fp4q_status status);
int fp4q_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FP4Q_H */
