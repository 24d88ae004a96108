// MXFP4 GEMM consumer on gfx950's block-scaled MFMA: C = A B^T, where A [m][k] and B
// [n][k] are row-wise MXFP4 (E2M1 codes, two per byte with element 2i in the low
// nibble, and one E8M0 scale per 32 elements along k), accumulated in fp32.
//
// Sources: the notes on NVIDIA's NVFP4 recipe (qiita.com/nishiha, section
// "NVFP4フロー図") describe the forward, data-gradient and weight-gradient products that
// consume the quantized operands; the FP4 glossary (ultralytics.com/ja/glossary/fp4,
// sections "FP4による推論と学習" and "FP4モデルのデプロイ") states that FP4 matrix products
// accumulate in higher precision and that MXFP4 runs natively on the MI350 family.
//
// v_mfma_scale_f32_32x32x64_f8f6f4 with both operands in E2M1 takes, per lane, 16
// bytes of codes (32 elements) and one E8M0 scale: lane l holds row l % 32 of its
// 32-row block and the 32-element K block l / 32 of the instruction's 64, for A and B
// alike; the 32 x 32 accumulator puts column l % 32 and rows 8(q/4) + 4(l/32) + q%4 in
// register q (checked with an in-bounds probe).  The order of the 32 elements inside a
// lane does not matter, since both operands use the same packing.
//
// Workgroup: a 256 x 256 tile of C, four waves of 128 x 128 (4 x 4 MFMA blocks, 256
// accumulator registers, one wave per SIMD).  A K step is 128 elements: 64 bytes of
// codes and one dword of four scales per row of each operand, copied straight into LDS
// by global_load_lds into one of four stages, so three steps are in flight while one
// is consumed.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "fp4q_internal.hpp"

namespace fp4q {
namespace {

typedef int v8i_t __attribute__((ext_vector_type(8)));
typedef float v16f_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_g __attribute__((ext_vector_type(4)));

constexpr int kGemmTile = 256;     // rows of A and of B per workgroup tile
constexpr int kGemmStages = 4;
constexpr int kLoadsPerStep = 10;  // global_load_lds per wave and K step: 4 + 4 code chunks, 2 scale words

struct GemmStage {
  u32x4_g a[kGemmTile * 4];   // 256 rows x four 16-byte chunks (swizzled)
  u32x4_g b[kGemmTile * 4];
  uint32_t as[kGemmTile];     // the four scales of each row for this K step
  uint32_t bs[kGemmTile];
};

// 16-byte chunk c of staged row r sits at position c ^ swz(r).  A fragment read takes
// 16 consecutive rows at one chunk; with this swizzle (a function of r % 16) their
// chunks fall in distinct bank groups whether LDS serves 8 or 16 such lanes per pass.
__device__ __forceinline__ uint32_t gemm_swz(uint32_t r) {
  return ((r >> 2) & 1u) | ((((r >> 1) ^ (r >> 3)) & 1u) << 1);
}

// Workgroup barrier that leaves the later steps' loads in flight (a memory fence would
// wait for all of them).  What it has to order is explicit: each wave has waited for
// its own loads of the step about to be read (wait_vm), and every read of the stage
// about to be refilled fed an MFMA of the previous step, so it has completed.
__device__ __forceinline__ void gemm_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

template <int N>
__device__ __forceinline__ void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Workgroup b -> C tile.  The blocks an XCD runs (b % 8 == x) take one contiguous range
// of the tile order, and that order walks groups of four tile rows column by column,
// so the tiles resident on one XCD share A rows and B rows in its L2.
__device__ __forceinline__ void gemm_tile(int b, int tiles_m, int tiles_n, int& tm, int& tn) {
  const int total = tiles_m * tiles_n;
  const int q = total >> 3, r = total & 7, x = b & 7;
  const int t = x * q + min(x, r) + (b >> 3);
  constexpr int G = 4;
  const int group = t / (G * tiles_n);
  const int first = group * G;
  const int gh = min(G, tiles_m - first);
  const int rem = t - group * G * tiles_n;
  tn = rem / gh;
  tm = first + rem % gh;
}

__device__ __forceinline__ uint16_t bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

template <int SUB>
__device__ __forceinline__ void gemm_substep(const GemmStage& s, uint32_t offA, uint32_t offB, const uint32_t sa[4],
                                             const uint32_t sb[4], v16f_t acc[4][4]) {
  v8i_t a[4], b[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const u32x4_g va = *reinterpret_cast<const u32x4_g*>(reinterpret_cast<const char*>(s.a) + offA + i * 32 * 64);
    const u32x4_g vb = *reinterpret_cast<const u32x4_g*>(reinterpret_cast<const char*>(s.b) + offB + i * 32 * 64);
    a[i] = v8i_t{(int)va.x, (int)va.y, (int)va.z, (int)va.w, 0, 0, 0, 0};
    b[i] = v8i_t{(int)vb.x, (int)vb.y, (int)vb.z, (int)vb.w, 0, 0, 0, 0};
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[i], b[j], acc[i][j], 4, 4, 2 * SUB, (int)sa[i],
                                                                  2 * SUB, (int)sb[j]);
}

template <bool BF16OUT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void k_gemm_mxfp4(
    const uint8_t* __restrict__ ac, const uint8_t* __restrict__ as, const uint8_t* __restrict__ bc,
    const uint8_t* __restrict__ bs, int M, int N, int K, int tiles_m, int tiles_n, void* __restrict__ cout) {
  __shared__ GemmStage st[kGemmStages];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  int tm, tn;
  gemm_tile(blockIdx.x, tiles_m, tiles_n, tm, tn);
  const int m0 = tm * kGemmTile, n0 = tn * kGemmTile;
  const int64_t ldq = K / 2, lds = K / 32;   // row strides of codes and scales, bytes
  const int nk = K / 128;

  // Loader: chunk p = 256 j + tid of a stage is row 64 j + tid / 4, position tid % 4,
  // which holds global chunk (tid % 4) ^ swz(row); rows past the matrix read its last
  // row (their products land in C rows or columns that are not stored).
  const int lr = tid >> 2;
  const uint32_t gch = (uint32_t)(tid & 3) ^ gemm_swz((uint32_t)lr);
  const uint8_t* pa[4];
  const uint8_t* pb[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    pa[j] = ac + (int64_t)min(m0 + 64 * j + lr, M - 1) * ldq + gch * 16;
    pb[j] = bc + (int64_t)min(n0 + 64 * j + lr, N - 1) * ldq + gch * 16;
  }
  const uint8_t* psa = as + (int64_t)min(m0 + tid, M - 1) * lds;
  const uint8_t* psb = bs + (int64_t)min(n0 + tid, N - 1) * lds;

  auto issue = [&](int ks) {
    GemmStage& s = st[ks % kGemmStages];
    const int64_t ko = (int64_t)ks * 64, so = (int64_t)ks * 4;
#pragma unroll
    for (int j = 0; j < 4; ++j) __builtin_amdgcn_global_load_lds(pa[j] + ko, &s.a[j * 256 + wave * 64], 16, 0, 0);
#pragma unroll
    for (int j = 0; j < 4; ++j) __builtin_amdgcn_global_load_lds(pb[j] + ko, &s.b[j * 256 + wave * 64], 16, 0, 0);
    __builtin_amdgcn_global_load_lds(psa + so, &s.as[wave * 64], 4, 0, 0);
    __builtin_amdgcn_global_load_lds(psb + so, &s.bs[wave * 64], 4, 0, 0);
  };

  // Fragment reads: row wm*128 + 32 i + fr, chunk (2 sub + fh) ^ swz(fr).
  const int wm = wave & 1, wn = wave >> 1;
  const int fr = lane & 31, fh = lane >> 5;
  const uint32_t sw = gemm_swz((uint32_t)fr);
  const uint32_t rowA = (uint32_t)(wm * 128 + fr) * 64, rowB = (uint32_t)(wn * 128 + fr) * 64;
  const uint32_t pos0 = (((uint32_t)fh) ^ sw) * 16, pos1 = (((uint32_t)(2 + fh)) ^ sw) * 16;

  v16f_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = v16f_t{};

#pragma unroll
  for (int p = 0; p < kGemmStages - 1; ++p)
    if (p < nk) issue(p);

  for (int ks = 0; ks < nk; ++ks) {
    // Step ks has landed once at most the loads of the steps issued after it remain.
    const int after = min(kGemmStages - 2, nk - 1 - ks);
    if (after >= 2) wait_vm<2 * kLoadsPerStep>();
    else if (after == 1) wait_vm<kLoadsPerStep>();
    else wait_vm<0>();
    gemm_barrier();    // every wave's share of step ks is in LDS; step ks-1's stage is free
    if (ks + kGemmStages - 1 < nk) issue(ks + kGemmStages - 1);

    const GemmStage& s = st[ks % kGemmStages];
    uint32_t sa[4], sb[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      sa[i] = s.as[wm * 128 + 32 * i + fr] >> (8 * fh);   // byte 2 sub of the shifted word: block 2 sub + fh
      sb[i] = s.bs[wn * 128 + 32 * i + fr] >> (8 * fh);
    }
    gemm_substep<0>(s, rowA + pos0, rowB + pos0, sa, sb, acc);
    gemm_substep<1>(s, rowA + pos1, rowB + pos1, sa, sb, acc);
  }

  // Epilogue: register q of block (i, j) is C row m0 + wm*128 + 32 i + 8(q/4) + 4 fh + q%4,
  // column n0 + wn*128 + 32 j + fr.
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int col = n0 + wn * 128 + 32 * j + fr;
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int row = m0 + wm * 128 + 32 * i + 8 * (q >> 2) + 4 * fh + (q & 3);
        if (row < M && col < N) {
          const int64_t o = (int64_t)row * N + col;
          if constexpr (BF16OUT)
            static_cast<uint16_t*>(cout)[o] = bf16_rne(acc[i][j][q]);
          else
            static_cast<float*>(cout)[o] = acc[i][j][q];
        }
      }
    }
  }
}

}  // namespace

bool launch_gemm_mxfp4(const uint8_t* ac, const uint8_t* as, const uint8_t* bc, const uint8_t* bs, int64_t m,
                       int64_t n, int64_t k, bool bf16_out, void* c, hipStream_t st) {
  const int tiles_m = (int)((m + kGemmTile - 1) / kGemmTile), tiles_n = (int)((n + kGemmTile - 1) / kGemmTile);
  const int64_t total = (int64_t)tiles_m * tiles_n;
  if (total > 0x7FFFFFFF) return false;
  if (bf16_out)
    k_gemm_mxfp4<true><<<(unsigned)total, 256, 0, st>>>(ac, as, bc, bs, (int)m, (int)n, (int)k, tiles_m, tiles_n, c);
  else
    k_gemm_mxfp4<false><<<(unsigned)total, 256, 0, st>>>(ac, as, bc, bs, (int)m, (int)n, (int)k, tiles_m, tiles_n, c);
  return true;
}

}  // namespace fp4q
