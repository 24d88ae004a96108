// fp4q_internal.hpp -- launchers shared between the C-ABI layer and the kernel files.
// Every launcher enqueues on `st` and assumes its arguments were validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp4q {

constexpr int kFusedMaxWg = 2048;
constexpr int kAmaxSpread = 128;   // cache lines an amax-reporting pass spreads its posts over

// Device-side state of a two-pass call (an amax pass A, then a quantizer Q) kept in a
// caller's workspace, so that nothing is numbered on the host and a call captured in
// a graph stays correct on every replay.  A reads `ea`, posts its workgroup maxima by
// atomic max into slot[ea & 1], and one of its threads records ea in `eq` and clears
// the other slot for the next call; Q reads slot[eq & 1] and one of its threads
// advances ea to eq + 1.  No kernel writes a word that its own workgroups read, and
// every word is consumed one kernel boundary after it is written.
struct alignas(128) TwoPassAmax {
  uint32_t ea;
  uint32_t pad0[31];
  uint32_t eq;
  uint32_t pad1[31];
  uint32_t slot[2][32];   // float bits (magnitudes), one 128-byte line each
};

// The one-pass kernel's exchange: per group of workgroups its members' slots and the
// group maximum, as (epoch << 32) | float bits, plus a count of waits that ran out.
struct FusedArea {
  uint64_t local[8][kFusedMaxWg / 8 + 16];
  uint64_t group[8][16];
  uint32_t fallbacks[32];
};

// Device memory of a workspace.  Every word starts at zero.
struct WorkspaceMem {
  FusedArea fused;
  TwoPassAmax two_pass;
  uint32_t spread[kAmaxSpread][32];   // MXFP4's amax report: zero between calls
};

// Where an amax pass posts (a float the call zeroed first, or a workspace's two-pass
// slot) and where a quantizer reads the tensor amax from (device side in fp4q_dev.hpp).
struct AmaxSink {
  float* f;
  TwoPassAmax* tp;
};
struct AmaxSource {
  const float* f;     // tensor amax given by the caller (or posted into it), or
  TwoPassAmax* tp;    // the slot an amax pass of the same call posted into
  float* out;         // with `tp`: the caller's amax output, written by one thread
};

// amax of x into a zeroed-first float (the standalone entry point) or a sink
void launch_amax(const void* x, int dtype, int64_t n, float* amax, hipStream_t st);
void launch_amax_to(const void* x, int dtype, int64_t n, const AmaxSink& sink, hipStream_t st);

void launch_nvfp4(const void* x, int dtype, int64_t rows, int64_t cols, unsigned layouts, bool sr,
                  const AmaxSource& amax, float* tensor_scale, uint8_t* row_codes, uint8_t* row_scales,
                  uint8_t* col_codes, uint8_t* col_scales, uint64_t seed, hipStream_t st);

// NVFP4 with amax computed in the same pass, through the workspace's exchange area
// with launch number `epoch`.  Returns false, having enqueued nothing, when the tensor
// does not fit one co-resident grid.  `wait_iters` bounds each wait (polls of >= 0.1 us).
bool launch_nvfp4_fused(const void* x, int dtype, int64_t rows, int64_t cols, unsigned layouts, bool sr,
                        float* amax, float* tensor_scale, uint8_t* row_codes, uint8_t* row_scales,
                        uint8_t* col_codes, uint8_t* col_scales, uint64_t seed, FusedArea* area, uint32_t epoch,
                        uint32_t wait_iters, hipStream_t st);
// Clears a workspace's exchange area, or any 4-byte aligned range, on the stream (a fill
// kernel, no memset node).
void launch_clear_fused(FusedArea* area, hipStream_t st);
void launch_clear_scratch(void* p, int64_t bytes, hipStream_t st);

void launch_nvfp4_2d(const void* x, int dtype, int64_t rows, int64_t cols, const AmaxSource& amax,
                     float* tensor_scale, uint8_t* codes, uint8_t* scales, uint8_t* codes_t, hipStream_t st);

// amax: NULL, or a device float that receives max|x| over the tensor; the workgroups
// post into the workspace's spread lines and a second, one-workgroup launch folds them
// (and clears them for the next call).
void launch_mxfp4(const void* x, int dtype, int64_t rows, int64_t cols, bool sr, uint8_t* codes,
                  uint8_t* scales, uint64_t seed, float* amax, uint32_t* spread, hipStream_t st);

void launch_if4(const void* x, int dtype, int64_t rows, int64_t cols, const AmaxSource& amax,
                float* tensor_scale, uint8_t* codes, uint8_t* scales, hipStream_t st);

void launch_dequant(int fmt, const uint8_t* codes, const uint8_t* scales, const float* tensor_scale,
                    int64_t rows, int64_t cols, int out_dtype, void* y, hipStream_t st);

// Random Hadamard transform along rows (chunks of 128) -- fp4q_rht.hip.
void launch_rht(const void* x, int dtype, int64_t rows, int64_t cols, const uint32_t signs[4],
                int inverse, float* y, hipStream_t st);
// x is bf16 (MFMA contraction) or, with f32, fp32 (VALU butterflies).
void launch_rht_amax(const void* x, bool f32, int64_t rows, int64_t cols, const uint32_t signs[4],
                     const AmaxSink& sink, hipStream_t st);
void launch_rht_nvfp4_col(const void* x, bool f32, int64_t rows, int64_t cols, const uint32_t signs[4],
                          bool sr, uint64_t seed, const AmaxSource& amax, float* tensor_scale,
                          uint8_t* col_codes, uint8_t* col_scales, hipStream_t st);

// Block-format variants (0 Four Over Six, 1 NVINT4, 2 IF3, 3 IF4, 4 IF6) -- fp4q_variant.hip.
void launch_variant(int var, const void* x, int dtype, int64_t rows, int64_t cols, const AmaxSource& amax,
                    float* tensor_scale, uint8_t* codes, uint8_t* scales, hipStream_t st);
void launch_dequant_variant(int var, const uint8_t* codes, const uint8_t* scales, const float* tensor_scale,
                            int64_t rows, int64_t cols, int out_dtype, void* y, hipStream_t st);

// MX FP6 (fmt 0 E2M3, 1 E3M2) quantize and dequantize -- fp4q_quant.hip.
void launch_mxfp6(const void* x, int dtype, int64_t rows, int64_t cols, int fmt, uint8_t* codes, uint8_t* scales,
                  hipStream_t st);
void launch_dequant_mxfp6(int fmt, const uint8_t* codes, const uint8_t* scales, int64_t rows, int64_t cols,
                          int out_dtype, void* y, hipStream_t st);

// MXFP4 GEMM C = A B^T (fp32 accumulate; fp32 or bf16 out) -- fp4q_gemm.hip.  k % 128 == 0.
// Both GEMMs write max |C| over the stored (rounded) outputs to `amax` when it is not null.
bool launch_gemm_mxfp4(const uint8_t* a_codes, const uint8_t* a_scales, const uint8_t* b_codes,
                       const uint8_t* b_scales, int64_t m, int64_t n, int64_t k, bool bf16_out, void* c,
                       float* amax, hipStream_t st);
// NVFP4 1x16 GEMM C = A B^T / (gs_a gs_b) on the f16 / bf16 MFMA -- fp4q_gemm.hip.  k % 128 == 0.
// flags bit 0 / bit 1: A / B carries 16x16 scale tiles ([rows/16][k/16]) instead of 1x16;
// bit 2 / bit 3: A / B is IF4 (scale bit 7 marks INT4 blocks).
bool launch_gemm_nvfp4(const uint8_t* a_codes, const uint8_t* a_scales, const float* a_ts, const uint8_t* b_codes,
                       const uint8_t* b_scales, const float* b_ts, int64_t m, int64_t n, int64_t k, bool bf16_out,
                       void* c, float* amax, unsigned flags, hipStream_t st);

}  // namespace fp4q
