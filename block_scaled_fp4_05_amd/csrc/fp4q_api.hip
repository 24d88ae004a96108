// fp4q_api.hip -- the extern "C" entry points of libfp4q: argument validation on the
// host, then kernel launches on the caller's stream.  See include/fp4q.h for the
// contract of each call.
#include "../../include/fp4q.h"
#include "fp4q_internal.hpp"

#include <mutex>
#include <new>
#include <stdint.h>

// The caller-owned workspace handle: the device memory and the host's numbering of
// one-pass launches on it.
struct fp4q_workspace {
  int device;
  fp4q::WorkspaceMem* mem;
  uint32_t epoch;        // one-pass launches enqueued so far; device slots start at epoch 0
  uint32_t wait_iters;   // polls of >= 0.1 us before a one-pass wait gives up
};
static_assert(sizeof(fp4q::WorkspaceMem) <= FP4Q_WORKSPACE_BYTES, "workspace size in fp4q.h is too small");

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }
bool valid_dtype(int d) { return d == FP4Q_F32 || d == FP4Q_BF16; }
bool valid_round(int r) { return r == FP4Q_RTN || r == FP4Q_SR; }

// Sink of a two-pass call's amax pass and the matching source for its quantizer: the
// workspace's two-pass state when there is one, else the caller's float (which the
// amax pass zeroes first).
fp4q::AmaxSink amax_sink(float* amax, fp4q_workspace* ws, fp4q::AmaxSource* src) {
  if (ws) {
    fp4q::TwoPassAmax* tp = &ws->mem->two_pass;
    *src = fp4q::AmaxSource{nullptr, tp, amax};
    return fp4q::AmaxSink{nullptr, tp};
  }
  *src = fp4q::AmaxSource{amax, nullptr, nullptr};
  return fp4q::AmaxSink{amax, nullptr};
}

// A workspace must be used on the device it lives on.
bool ws_ok(const fp4q_workspace* ws) {
  if (!ws) return true;
  int dev = -1;
  return hipGetDevice(&dev) == hipSuccess && dev == ws->device;
}

// Whether work enqueued on `st` is being captured into a graph (then the one-pass
// kernel, whose launch number is a host value, is not used).
bool capturing(hipStream_t st) {
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(st, &cs) != hipSuccess) return true;   // unknown: take the safe path
  return cs != hipStreamCaptureStatusNone;
}

fp4q_status after_launch() {
  return hipGetLastError() == hipSuccess ? FP4Q_OK : FP4Q_E_HIP;
}

// Host Philox4x32-10 for the RHT sign mask (Salmon et al., SC'11).
void philox4x32_10_host(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]) {
  uint32_t c[4] = {ctr[0], ctr[1], ctr[2], ctr[3]};
  uint32_t k0 = key[0], k1 = key[1];
  for (int r = 0; r < 10; ++r) {
    const uint64_t p0 = (uint64_t)0xD2511F53u * c[0];
    const uint64_t p1 = (uint64_t)0xCD9E8D57u * c[2];
    const uint32_t n0 = (uint32_t)(p1 >> 32) ^ c[1] ^ k0;
    const uint32_t n2 = (uint32_t)(p0 >> 32) ^ c[3] ^ k1;
    c[1] = (uint32_t)p1;
    c[3] = (uint32_t)p0;
    c[0] = n0;
    c[2] = n2;
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
  for (int i = 0; i < 4; ++i) out[i] = c[i];
}

// Argument checks of fp4q_quantize_nvfp4 (and of its allocation-free form).
fp4q_status check_nvfp4(const void* x, fp4q_dtype dt, int64_t rows, int64_t cols, unsigned layouts, fp4q_round rnd,
                        const uint32_t* rht_signs, unsigned amax_mode, const float* amax, const float* tensor_scale,
                        const uint8_t* row_codes, const uint8_t* row_scales, const uint8_t* col_codes,
                        const uint8_t* col_scales) {
  const bool row = (layouts & FP4Q_ROWWISE) != 0, col = (layouts & FP4Q_COLWISE) != 0;
  if (!x || !amax || !tensor_scale) return FP4Q_E_NULL;
  if (row && (!row_codes || !row_scales)) return FP4Q_E_NULL;
  if (col && (!col_codes || !col_scales)) return FP4Q_E_NULL;
  if (!valid_dtype(dt) || !valid_round(rnd) || layouts == 0 || (layouts & ~3u) != 0 ||
      (amax_mode != FP4Q_AMAX_COMPUTE && amax_mode != FP4Q_AMAX_GIVEN))
    return FP4Q_E_ARG;
  if (rht_signs && layouts != FP4Q_COLWISE) return FP4Q_E_ARG;
  if (rows <= 0 || cols <= 0 || rows > INT32_MAX || cols > INT32_MAX) return FP4Q_E_SHAPE;
  if (row && cols % 16 != 0) return FP4Q_E_SHAPE;
  if (col && (rows % 16 != 0 || cols % 8 != 0)) return FP4Q_E_SHAPE;
  if (rht_signs && (rows % 128 != 0 || cols >= (int64_t(1) << 27))) return FP4Q_E_SHAPE;
  if (!aligned16(x) || !aligned4(amax) || !aligned4(tensor_scale)) return FP4Q_E_ALIGN;
  if (row && (!aligned16(row_codes) || !aligned16(row_scales))) return FP4Q_E_ALIGN;
  if (col && (!aligned16(col_codes) || !aligned16(col_scales))) return FP4Q_E_ALIGN;
  return FP4Q_OK;
}

}  // namespace

extern "C" {

int fp4q_abi_version(void) { return FP4Q_ABI_VERSION; }

const char* fp4q_status_string(fp4q_status s) {
  switch (s) {
    case FP4Q_OK: return "ok";
    case FP4Q_E_NULL: return "a required pointer is NULL";
    case FP4Q_E_SHAPE: return "shape is not a positive multiple of the block size";
    case FP4Q_E_ALIGN: return "a device pointer is not 16-byte aligned";
    case FP4Q_E_ARG: return "invalid argument or unsupported combination";
    case FP4Q_E_HIP: return "HIP runtime error while enqueueing";
  }
  return "unknown status";
}

fp4q_status fp4q_workspace_create(fp4q_workspace** ws) {
  if (!ws) return FP4Q_E_NULL;
  *ws = nullptr;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return FP4Q_E_HIP;
  void* mem = nullptr;
  if (hipMalloc(&mem, FP4Q_WORKSPACE_BYTES) != hipSuccess) return FP4Q_E_HIP;
  if (hipMemset(mem, 0, FP4Q_WORKSPACE_BYTES) != hipSuccess || hipDeviceSynchronize() != hipSuccess) {
    (void)hipFree(mem);
    return FP4Q_E_HIP;
  }
  fp4q_workspace* w = new (std::nothrow) fp4q_workspace{dev, static_cast<fp4q::WorkspaceMem*>(mem), 0u, 2000u};
  if (!w) {
    (void)hipFree(mem);
    return FP4Q_E_HIP;
  }
  *ws = w;
  return FP4Q_OK;
}

fp4q_status fp4q_workspace_destroy(fp4q_workspace* ws) {
  if (!ws) return FP4Q_E_NULL;
  const hipError_t e = hipFree(ws->mem);
  delete ws;
  return e == hipSuccess ? FP4Q_OK : FP4Q_E_HIP;
}

fp4q_status fp4q_workspace_set_wait(fp4q_workspace* ws, uint32_t microseconds) {
  if (!ws) return FP4Q_E_NULL;
  const uint64_t t = (uint64_t)microseconds * 10u;   // one poll round takes at least ~0.1 us
  ws->wait_iters = t > 0xFFFFFFFFull ? 0xFFFFFFFFu : (uint32_t)t;
  return FP4Q_OK;
}

fp4q_status fp4q_workspace_fallbacks(fp4q_workspace* ws, hipStream_t stream, uint32_t* count) {
  if (!ws || !count) return FP4Q_E_NULL;
  if (!ws_ok(ws)) return FP4Q_E_ARG;
  return hipMemcpyAsync(count, &ws->mem->fused.fallbacks[0], 4, hipMemcpyDeviceToHost, stream) == hipSuccess &&
                 hipStreamSynchronize(stream) == hipSuccess
             ? FP4Q_OK
             : FP4Q_E_HIP;
}

void fp4q_rht_signs_from_seed(uint64_t seed, uint32_t signs[4]) {
  const uint32_t ctr[4] = {0u, 0u, 0u, 1u};
  const uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
  philox4x32_10_host(ctr, key, signs);
}

fp4q_status fp4q_amax(const void* x, fp4q_dtype dt, int64_t rows, int64_t cols, float* amax, hipStream_t stream) {
  if (!x || !amax) return FP4Q_E_NULL;
  if (!valid_dtype(dt)) return FP4Q_E_ARG;
  if (rows <= 0 || cols <= 0) return FP4Q_E_SHAPE;
  if (!aligned16(x) || !aligned4(amax)) return FP4Q_E_ALIGN;
  fp4q::launch_amax(x, dt, rows * cols, amax, stream);
  return after_launch();
}

fp4q_status fp4q_quantize_nvfp4(const void* x, fp4q_dtype dt, int64_t rows, int64_t cols, unsigned layouts,
                                fp4q_round rnd, uint64_t sr_seed, const uint32_t* rht_signs, unsigned amax_mode,
                                float* amax, float* tensor_scale, uint8_t* row_codes, uint8_t* row_scales,
                                uint8_t* col_codes, uint8_t* col_scales, fp4q_workspace* ws, hipStream_t stream) {
  const fp4q_status v = check_nvfp4(x, dt, rows, cols, layouts, rnd, rht_signs, amax_mode, amax, tensor_scale,
                                    row_codes, row_scales, col_codes, col_scales);
  if (v != FP4Q_OK) return v;
  if (!ws_ok(ws)) return FP4Q_E_ARG;

  const bool sr = rnd == FP4Q_SR;
  if (rht_signs) {
    const bool f32 = dt == FP4Q_F32;
    fp4q::AmaxSource src{amax, nullptr, nullptr};
    if (amax_mode == FP4Q_AMAX_COMPUTE) {
      const fp4q::AmaxSink sink = amax_sink(amax, ws, &src);
      fp4q::launch_rht_amax(x, f32, rows, cols, rht_signs, sink, stream);
    }
    fp4q::launch_rht_nvfp4_col(x, f32, rows, cols, rht_signs, sr, sr_seed, src, tensor_scale, col_codes, col_scales,
                               stream);
    return after_launch();
  }
  fp4q::AmaxSource src{amax, nullptr, nullptr};
  if (amax_mode == FP4Q_AMAX_COMPUTE) {
    // one pass when the tensor fits a co-resident grid, else amax first
    if (ws && !capturing(stream)) {
      uint32_t epoch = ws->epoch + 1u;
      if (epoch == 0u) {
        // after 2^32 launches the numbers repeat: clear the exchange first, so no slot
        // left by an earlier launch can carry the current number
        fp4q::launch_clear_fused(&ws->mem->fused, stream);
        epoch = 1u;
      }
      if (fp4q::launch_nvfp4_fused(x, dt, rows, cols, layouts, sr, amax, tensor_scale, row_codes, row_scales,
                                   col_codes, col_scales, sr_seed, &ws->mem->fused, epoch, ws->wait_iters,
                                   stream)) {
        ws->epoch = epoch;
        return after_launch();
      }
    }
    fp4q::launch_amax_to(x, dt, rows * cols, amax_sink(amax, ws, &src), stream);
  }
  fp4q::launch_nvfp4(x, dt, rows, cols, layouts, sr, src, tensor_scale, row_codes, row_scales, col_codes,
                     col_scales, sr_seed, stream);
  return after_launch();
}

fp4q_status fp4q_quantize_nvfp4_2d(const void* x, fp4q_dtype dt, int64_t rows, int64_t cols, unsigned amax_mode,
                                   float* amax, float* tensor_scale, uint8_t* codes, uint8_t* scales,
                                   uint8_t* codes_t, fp4q_workspace* ws, hipStream_t stream) {
  if (!x || !amax || !tensor_scale || !codes || !scales) return FP4Q_E_NULL;
  if (!valid_dtype(dt) || (amax_mode != FP4Q_AMAX_COMPUTE && amax_mode != FP4Q_AMAX_GIVEN)) return FP4Q_E_ARG;
  if (rows <= 0 || cols <= 0 || rows % 16 != 0 || cols % 16 != 0) return FP4Q_E_SHAPE;
  if (!aligned16(x) || !aligned16(codes) || !aligned16(scales) || !aligned4(amax) || !aligned4(tensor_scale) ||
      (codes_t && !aligned16(codes_t)))
    return FP4Q_E_ALIGN;
  if (!ws_ok(ws)) return FP4Q_E_ARG;
  fp4q::AmaxSource src{amax, nullptr, nullptr};
  if (amax_mode == FP4Q_AMAX_COMPUTE) fp4q::launch_amax_to(x, dt, rows * cols, amax_sink(amax, ws, &src), stream);
  fp4q::launch_nvfp4_2d(x, dt, rows, cols, src, tensor_scale, codes, scales, codes_t, stream);
  return after_launch();
}

fp4q_status fp4q_quantize_mxfp4(const void* x, fp4q_dtype dt, int64_t rows, int64_t cols, fp4q_round rnd,
                                uint64_t sr_seed, uint8_t* codes, uint8_t* scales, float* amax,
                                fp4q_workspace* ws, hipStream_t stream) {
  if (!x || !codes || !scales || (amax && !ws)) return FP4Q_E_NULL;
  if (!valid_dtype(dt) || !valid_round(rnd)) return FP4Q_E_ARG;
  if (rows <= 0 || cols <= 0 || cols % 32 != 0) return FP4Q_E_SHAPE;
  if (!aligned16(x) || !aligned16(codes) || !aligned16(scales) || (amax && !aligned4(amax))) return FP4Q_E_ALIGN;
  if (!ws_ok(ws)) return FP4Q_E_ARG;
  fp4q::launch_mxfp4(x, dt, rows, cols, rnd == FP4Q_SR, codes, scales, sr_seed, amax,
                     ws ? &ws->mem->spread[0][0] : nullptr, stream);
  return after_launch();
}

fp4q_status fp4q_quantize_mxfp6(const void* x, fp4q_dtype dt, int64_t rows, int64_t cols, fp4q_fp6 fmt,
                                uint8_t* codes, uint8_t* scales, hipStream_t stream) {
  if (!x || !codes || !scales) return FP4Q_E_NULL;
  if (!valid_dtype(dt) || (fmt != FP4Q_FP6_E2M3 && fmt != FP4Q_FP6_E3M2)) return FP4Q_E_ARG;
  if (rows <= 0 || cols <= 0 || cols % 32 != 0) return FP4Q_E_SHAPE;
  if (!aligned16(x) || !aligned16(codes) || !aligned16(scales)) return FP4Q_E_ALIGN;
  fp4q::launch_mxfp6(x, dt, rows, cols, fmt == FP4Q_FP6_E3M2 ? 1 : 0, codes, scales, stream);
  return after_launch();
}

fp4q_status fp4q_quantize_if4(const void* x, fp4q_dtype dt, int64_t rows, int64_t cols, unsigned amax_mode,
                              float* amax, float* tensor_scale, uint8_t* codes, uint8_t* scales,
                              fp4q_workspace* ws, hipStream_t stream) {
  if (!x || !amax || !tensor_scale || !codes || !scales) return FP4Q_E_NULL;
  if (!valid_dtype(dt) || (amax_mode != FP4Q_AMAX_COMPUTE && amax_mode != FP4Q_AMAX_GIVEN)) return FP4Q_E_ARG;
  if (rows <= 0 || cols <= 0 || cols % 16 != 0) return FP4Q_E_SHAPE;
  if (!aligned16(x) || !aligned16(codes) || !aligned16(scales) || !aligned4(amax) || !aligned4(tensor_scale))
    return FP4Q_E_ALIGN;
  if (!ws_ok(ws)) return FP4Q_E_ARG;
  fp4q::AmaxSource src{amax, nullptr, nullptr};
  if (amax_mode == FP4Q_AMAX_COMPUTE) fp4q::launch_amax_to(x, dt, rows * cols, amax_sink(amax, ws, &src), stream);
  fp4q::launch_if4(x, dt, rows, cols, src, tensor_scale, codes, scales, stream);
  return after_launch();
}

fp4q_status fp4q_quantize_variant(const void* x, fp4q_dtype dt, int64_t rows, int64_t cols, fp4q_variant var,
                                  unsigned amax_mode, float* amax, float* tensor_scale, uint8_t* codes,
                                  uint8_t* scales, fp4q_workspace* ws, hipStream_t stream) {
  if (!x || !amax || !tensor_scale || !codes || !scales) return FP4Q_E_NULL;
  if (!valid_dtype(dt) || (int)var < 0 || (int)var > 4 ||
      (amax_mode != FP4Q_AMAX_COMPUTE && amax_mode != FP4Q_AMAX_GIVEN))
    return FP4Q_E_ARG;
  if (rows <= 0 || cols <= 0 || cols % 16 != 0) return FP4Q_E_SHAPE;
  if (!aligned16(x) || !aligned16(codes) || !aligned16(scales) || !aligned4(amax) || !aligned4(tensor_scale))
    return FP4Q_E_ALIGN;
  if (!ws_ok(ws)) return FP4Q_E_ARG;
  fp4q::AmaxSource src{amax, nullptr, nullptr};
  if (amax_mode == FP4Q_AMAX_COMPUTE) fp4q::launch_amax_to(x, dt, rows * cols, amax_sink(amax, ws, &src), stream);
  fp4q::launch_variant((int)var, x, dt, rows, cols, src, tensor_scale, codes, scales, stream);
  return after_launch();
}

fp4q_status fp4q_dequantize_variant(fp4q_variant var, const uint8_t* codes, const uint8_t* scales,
                                    const float* tensor_scale, int64_t rows, int64_t cols, fp4q_dtype out_dt,
                                    void* y, hipStream_t stream) {
  if (!codes || !scales || !tensor_scale || !y) return FP4Q_E_NULL;
  if ((int)var < 0 || (int)var > 4 || !valid_dtype(out_dt)) return FP4Q_E_ARG;
  if (rows <= 0 || cols <= 0 || cols % 16 != 0) return FP4Q_E_SHAPE;
  if (!aligned16(codes) || !aligned16(scales) || !aligned16(y) || !aligned4(tensor_scale)) return FP4Q_E_ALIGN;
  fp4q::launch_dequant_variant((int)var, codes, scales, tensor_scale, rows, cols, out_dt, y, stream);
  return after_launch();
}

fp4q_status fp4q_rht(const void* x, fp4q_dtype dt, int64_t rows, int64_t cols, const uint32_t* signs, int inverse,
                     float* y, hipStream_t stream) {
  if (!x || !signs || !y) return FP4Q_E_NULL;
  if (!valid_dtype(dt)) return FP4Q_E_ARG;
  if (rows <= 0 || cols <= 0 || rows % 128 != 0 || cols % 8 != 0) return FP4Q_E_SHAPE;
  if (!aligned16(x) || !aligned16(y)) return FP4Q_E_ALIGN;
  fp4q::launch_rht(x, dt, rows, cols, signs, inverse ? 1 : 0, y, stream);
  return after_launch();
}

fp4q_status fp4q_gemm_mxfp4(const uint8_t* a_codes, const uint8_t* a_scales, const uint8_t* b_codes,
                            const uint8_t* b_scales, int64_t m, int64_t n, int64_t k, fp4q_dtype out_dt, void* c,
                            float* amax, hipStream_t stream) {
  if (!a_codes || !a_scales || !b_codes || !b_scales || !c) return FP4Q_E_NULL;
  if (!valid_dtype(out_dt)) return FP4Q_E_ARG;
  const int64_t lim = (int64_t)1 << 31;
  if (m <= 0 || n <= 0 || k < 128 || k % 128 != 0 || m >= lim || n >= lim || k > ((int64_t)1 << 25))
    return FP4Q_E_SHAPE;
  if (!aligned16(a_codes) || !aligned16(a_scales) || !aligned16(b_codes) || !aligned16(b_scales) || !aligned16(c) ||
      !aligned4(amax))
    return FP4Q_E_ALIGN;
  if (!fp4q::launch_gemm_mxfp4(a_codes, a_scales, b_codes, b_scales, m, n, k, out_dt == FP4Q_BF16, c, amax, stream))
    return FP4Q_E_SHAPE;
  return after_launch();
}

fp4q_status fp4q_gemm_nvfp4(const uint8_t* a_codes, const uint8_t* a_scales, const float* a_tensor_scale,
                            const uint8_t* b_codes, const uint8_t* b_scales, const float* b_tensor_scale, int64_t m,
                            int64_t n, int64_t k, unsigned operand_flags, fp4q_dtype out_dt, void* c, float* amax,
                            hipStream_t stream) {
  if (!a_codes || !a_scales || !a_tensor_scale || !b_codes || !b_scales || !b_tensor_scale || !c) return FP4Q_E_NULL;
  const unsigned scale_tiles = operand_flags & 3u;
  if (!valid_dtype(out_dt) || (operand_flags & ~15u) != 0 ||
      ((operand_flags & FP4Q_TILES_A) && (operand_flags & FP4Q_IF4_A)) ||
      ((operand_flags & FP4Q_TILES_B) && (operand_flags & FP4Q_IF4_B)))
    return FP4Q_E_ARG;
  const int64_t lim = (int64_t)1 << 31;
  if (m <= 0 || n <= 0 || k < 128 || k % 128 != 0 || m >= lim || n >= lim || k > ((int64_t)1 << 25))
    return FP4Q_E_SHAPE;
  if (((scale_tiles & FP4Q_TILES_A) && m % 16 != 0) || ((scale_tiles & FP4Q_TILES_B) && n % 16 != 0))
    return FP4Q_E_SHAPE;
  if (!aligned16(a_codes) || !aligned16(a_scales) || !aligned16(b_codes) || !aligned16(b_scales) || !aligned16(c) ||
      !aligned4(a_tensor_scale) || !aligned4(b_tensor_scale) || !aligned4(amax))
    return FP4Q_E_ALIGN;
  if (!fp4q::launch_gemm_nvfp4(a_codes, a_scales, a_tensor_scale, b_codes, b_scales, b_tensor_scale, m, n, k,
                               out_dt == FP4Q_BF16, c, amax, operand_flags, stream))
    return FP4Q_E_SHAPE;
  return after_launch();
}

fp4q_status fp4q_dequantize(fp4q_format fmt, const uint8_t* codes, const uint8_t* scales, const float* tensor_scale,
                            int64_t rows, int64_t cols, fp4q_dtype out_dt, void* y, hipStream_t stream) {
  if (!codes || !scales || !y) return FP4Q_E_NULL;
  if (fmt == FP4Q_FMT_MXFP6_E2M3 || fmt == FP4Q_FMT_MXFP6_E3M2) {
    if (!valid_dtype(out_dt)) return FP4Q_E_ARG;
    if (rows <= 0 || cols <= 0 || cols % 32 != 0) return FP4Q_E_SHAPE;
    if (!aligned16(codes) || !aligned16(scales) || !aligned16(y)) return FP4Q_E_ALIGN;
    fp4q::launch_dequant_mxfp6(fmt == FP4Q_FMT_MXFP6_E3M2 ? 1 : 0, codes, scales, rows, cols, out_dt, y, stream);
    return after_launch();
  }
  if (fmt != FP4Q_FMT_NVFP4 && fmt != FP4Q_FMT_NVFP4_2D && fmt != FP4Q_FMT_MXFP4 && fmt != FP4Q_FMT_IF4)
    return FP4Q_E_ARG;
  if (!valid_dtype(out_dt)) return FP4Q_E_ARG;
  if (fmt != FP4Q_FMT_MXFP4 && !tensor_scale) return FP4Q_E_NULL;
  if (rows <= 0 || cols <= 0) return FP4Q_E_SHAPE;
  if (fmt == FP4Q_FMT_MXFP4 && cols % 32 != 0) return FP4Q_E_SHAPE;
  if (fmt != FP4Q_FMT_MXFP4 && cols % 16 != 0) return FP4Q_E_SHAPE;
  if (fmt == FP4Q_FMT_NVFP4_2D && rows % 16 != 0) return FP4Q_E_SHAPE;
  if (!aligned16(codes) || !aligned16(scales) || !aligned16(y) || (tensor_scale && !aligned4(tensor_scale)))
    return FP4Q_E_ALIGN;
  fp4q::launch_dequant(fmt, codes, scales, tensor_scale, rows, cols, out_dt, y, stream);
  return after_launch();
}

// ---------------------------------------------------------------------------------------
// Allocation-free NVFP4 entry point.  Its workspace is this file-scope device array (one
// copy per GPU, alive until the process ends), found once per device by
// hipGetSymbolAddress; host code uses only that address, never the array's name.
// ---------------------------------------------------------------------------------------
static __device__ __align__(256) unsigned char scratch[FP4Q_WORKSPACE_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
fp4q_workspace g_scratch_ws[kMaxDevices];
bool g_scratch_ready[kMaxDevices];

// The device's scratch as a workspace, set up on first use with the device current.
fp4q_workspace* scratch_workspace(hipStream_t stream, fp4q_status* err) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    *err = FP4Q_E_HIP;
    return nullptr;
  }
  if (!g_scratch_ready[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) {
      *err = FP4Q_E_HIP;
      return nullptr;
    }
    g_scratch_ws[dev] = fp4q_workspace{dev, static_cast<fp4q::WorkspaceMem*>(ptr), 0u, 2000u};
    // every word of a workspace starts at zero: clear it with a fill kernel, ordered
    // before this call's kernels on the caller's stream
    fp4q::launch_clear_scratch(ptr, FP4Q_WORKSPACE_BYTES, stream);
    if (hipGetLastError() != hipSuccess) {
      *err = FP4Q_E_HIP;
      return nullptr;
    }
    g_scratch_ready[dev] = true;
  }
  return &g_scratch_ws[dev];
}

}  // namespace

fp4q_status fp4q_quantize_nvfp4_noalloc(const void* x, fp4q_dtype dt, int64_t rows, int64_t cols, unsigned layouts,
                                        fp4q_round rnd, uint64_t sr_seed, const uint32_t* rht_signs,
                                        unsigned amax_mode, float* amax, float* tensor_scale, uint8_t* row_codes,
                                        uint8_t* row_scales, uint8_t* col_codes, uint8_t* col_scales,
                                        hipStream_t stream) {
  // arguments are checked before the scratch is set up, as the workspace form checks them
  const fp4q_status pre = check_nvfp4(x, dt, rows, cols, layouts, rnd, rht_signs, amax_mode, amax, tensor_scale,
                                      row_codes, row_scales, col_codes, col_scales);
  if (pre != FP4Q_OK) return pre;
  std::lock_guard<std::mutex> lock(g_scratch_mu);   // the launch numbering of the device's scratch
  fp4q_status err = FP4Q_OK;
  fp4q_workspace* ws = scratch_workspace(stream, &err);
  if (!ws) return err;
  return fp4q_quantize_nvfp4(x, dt, rows, cols, layouts, rnd, sr_seed, rht_signs, amax_mode, amax, tensor_scale,
                             row_codes, row_scales, col_codes, col_scales, ws, stream);
}

}  // extern "C"
