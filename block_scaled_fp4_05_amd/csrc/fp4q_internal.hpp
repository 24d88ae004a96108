// fp4q_internal.hpp -- launchers shared between the C-ABI layer and the kernel files.
// Every launcher enqueues on `st` and assumes its arguments were validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp4q {

// Where an amax pass posts (a zeroed float, or a per-stream workspace word with an
// epoch) and where a quantizer reads the tensor amax from (device side in fp4q_dev.hpp).
struct AmaxSink {
  float* f;
  uint64_t* slot;
  uint32_t epoch;
};
struct AmaxSource {
  const float* f;         // tensor amax given by the caller, or
  const uint64_t* slot;   // the word an amax pass of the same stream posted into
  float* out;             // with `slot`: the caller's amax output, written by one thread
};

// amax of x into a zeroed-first float (the standalone entry point) or a sink
void launch_amax(const void* x, int dtype, int64_t n, float* amax, hipStream_t st);
void launch_amax_to(const void* x, int dtype, int64_t n, const AmaxSink& sink, hipStream_t st);
// The stream's workspace word for a two-pass call and the call's epoch (false if the
// workspace cannot be allocated; callers then use the caller's float instead).
bool reserve_amax_slot(hipStream_t st, uint64_t** slot, uint32_t* epoch);

void launch_nvfp4(const void* x, int dtype, int64_t rows, int64_t cols, unsigned layouts, bool sr,
                  const AmaxSource& amax, float* tensor_scale, uint8_t* row_codes, uint8_t* row_scales,
                  uint8_t* col_codes, uint8_t* col_scales, uint64_t seed, hipStream_t st);

// NVFP4 with amax computed in the same pass.  Returns false, having enqueued nothing,
// when the tensor does not fit one co-resident grid.
bool launch_nvfp4_fused(const void* x, int dtype, int64_t rows, int64_t cols, unsigned layouts, bool sr,
                        float* amax, float* tensor_scale, uint8_t* row_codes, uint8_t* row_scales,
                        uint8_t* col_codes, uint8_t* col_scales, uint64_t seed, hipStream_t st);
// Wait limit of the one-pass kernel's exchange before a workgroup computes a missing
// maximum itself, and the count of such fallbacks on a stream (synchronizes it).
void set_fused_wait_us(uint32_t us);
bool fused_fallbacks(hipStream_t st, uint32_t* count);
constexpr int kFusedMaxWg = 2048;
constexpr int kAmaxSpread = 128;   // cache lines an amax-reporting pass spreads its posts over

void launch_nvfp4_2d(const void* x, int dtype, int64_t rows, int64_t cols, const AmaxSource& amax,
                     float* tensor_scale, uint8_t* codes, uint8_t* scales, uint8_t* codes_t, hipStream_t st);

// amax: NULL, or a device float that receives max|x| over the tensor (a second,
// one-workgroup launch folds the workgroups' spread posts).  False if the per-stream
// workspace could not be set up (nothing launched then).
bool launch_mxfp4(const void* x, int dtype, int64_t rows, int64_t cols, bool sr, uint8_t* codes,
                  uint8_t* scales, uint64_t seed, float* amax, hipStream_t st);

void launch_if4(const void* x, int dtype, int64_t rows, int64_t cols, const AmaxSource& amax,
                float* tensor_scale, uint8_t* codes, uint8_t* scales, hipStream_t st);

void launch_dequant(int fmt, const uint8_t* codes, const uint8_t* scales, const float* tensor_scale,
                    int64_t rows, int64_t cols, int out_dtype, void* y, hipStream_t st);

// Random Hadamard transform along rows (chunks of 128) -- fp4q_rht.hip.
void launch_rht(const void* x, int dtype, int64_t rows, int64_t cols, const uint32_t signs[4],
                int inverse, float* y, hipStream_t st);
void launch_rht_amax(const uint16_t* x, int64_t rows, int64_t cols, const uint32_t signs[4],
                     const AmaxSink& sink, hipStream_t st);
void launch_rht_nvfp4_col(const uint16_t* x, int64_t rows, int64_t cols, const uint32_t signs[4],
                          bool sr, uint64_t seed, const AmaxSource& amax, float* tensor_scale,
                          uint8_t* col_codes, uint8_t* col_scales, hipStream_t st);

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
// NVFP4 1x16 GEMM C = A B^T / (gs_a gs_b) on the bf16 MFMA -- fp4q_gemm.hip.  k % 128 == 0.
bool launch_gemm_nvfp4(const uint8_t* a_codes, const uint8_t* a_scales, const float* a_ts, const uint8_t* b_codes,
                       const uint8_t* b_scales, const float* b_ts, int64_t m, int64_t n, int64_t k, bool bf16_out,
                       void* c, float* amax, hipStream_t st);

}  // namespace fp4q
