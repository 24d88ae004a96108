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
// accumulator registers, one wave per SIMD).  A K step is 256 elements: 128 bytes of
// codes per row of each operand, copied straight into LDS by global_load_lds into one
// of two stages while the other is consumed, plus the scales in chunks of two steps.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <type_traits>

#include "fp4q_internal.hpp"

namespace fp4q {
namespace {

typedef int v8i_t __attribute__((ext_vector_type(8)));
typedef float v16f_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_g __attribute__((ext_vector_type(4)));

constexpr int kGemmTile = 256;     // rows of A and of B per workgroup tile
constexpr int kGemmStages = 2;
constexpr int kLoadsPerStep = 20;  // global_load_lds per wave and K step: 8 + 8 code chunks, 4 scale slices

// A K step is 256 elements, 128 bytes of codes per row, so every load fetches whole
// 128-byte lines: with 64 bytes per row and step, each line was fetched twice (once
// per step) and the L2-to-LDS stream ran about 40 % slower.
struct GemmStage {
  u32x4_g a[kGemmTile * 8];   // 256 rows x eight 16-byte chunks (swizzled)
  u32x4_g b[kGemmTile * 8];
};

// Scales travel in chunks of two K steps: 16 bytes per row, eight E8M0 bytes per step.
// Row-major input keeps a row's scales for consecutive steps together, so one access
// per row brings two steps; a word per row and step would touch a cache line per row
// every time.  Three chunk buffers; the chunk for steps 2C and 2C+1 is loaded in four
// slices of 64 rows, two with the code loads of step 2C-2 and two with those of step
// 2C-1, so every step issues the same number of loads.  Word d of a row's 16 bytes
// (d = 2 (step % 2) + half of the step) sits at position d ^ scale_swz(row), which
// spreads 32 consecutive rows over distinct banks.
struct GemmScales {
  uint32_t a[kGemmTile * 4];
  uint32_t b[kGemmTile * 4];
};
__device__ __forceinline__ uint32_t scale_swz(uint32_t r) { return (r >> 3) & 3u; }

struct GemmLds {
  GemmStage st[kGemmStages];
  GemmScales sc[3];
};

// 16-byte chunk c of staged row r sits at position c ^ gemm_swz(r).  A fragment read
// takes 16 consecutive rows at one chunk; with this swizzle (a function of r % 16) they
// fall in distinct bank groups whether LDS serves 8 or 16 such lanes per pass.
__device__ __forceinline__ uint32_t gemm_swz(uint32_t r) {
  return ((r >> 1) & 1u) | (((r >> 2) & 1u) << 1) | (((r ^ (r >> 3)) & 1u) << 2);
}

// Workgroup barrier that leaves the next step's loads in flight (a memory fence would
// wait for all of them).  What it has to order is explicit: each wave has waited for
// its own loads of the step about to be read (wait_vm), and every read of the stage
// about to be refilled has completed (the LDS wait).  The LDS wait goes through the
// builtin so that the compiler's own wait insertion knows every earlier LDS read is done.
__device__ __forceinline__ void gemm_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0); vmcnt and expcnt at their maximum (no wait)
  asm volatile("s_barrier" ::: "memory");
}

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

// Output amax: each lane keeps the largest magnitude it stored as fp32 bits (a bf16 h
// widens exactly to h << 16), which order as unsigned integers as the values do; the wave
// folds them and one lane posts an atomic max, so a launch makes one atomic per wave.
// This is the tensor amax that a following amax-scaled quantization of C can be given.
__device__ __forceinline__ void post_amax(uint32_t m, uint32_t* amax) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, off, 64));
  if ((threadIdx.x & 63) == 0 && m) __hip_atomic_fetch_max(amax, m, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ uint32_t bf16x2_absmax(uint32_t w) {
  return max(w & 0x7FFFu, (w >> 16) & 0x7FFFu);
}

__global__ void k_gemm_amax_zero(uint32_t* p) { *p = 0u; }

// One 64-element K sub-step of a wave's 128 x 128 block: the 4 A and 4 B fragments.
struct GemmFrags {
  v8i_t a[4], b[4];
};

__device__ __forceinline__ void gemm_read(const GemmStage& s, uint32_t offA, uint32_t offB, GemmFrags& f) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const u32x4_g va = *reinterpret_cast<const u32x4_g*>(reinterpret_cast<const char*>(s.a) + offA + i * 32 * 128);
    const u32x4_g vb = *reinterpret_cast<const u32x4_g*>(reinterpret_cast<const char*>(s.b) + offB + i * 32 * 128);
    f.a[i] = v8i_t{(int)va.x, (int)va.y, (int)va.z, (int)va.w, 0, 0, 0, 0};
    f.b[i] = v8i_t{(int)vb.x, (int)vb.y, (int)vb.z, (int)vb.w, 0, 0, 0, 0};
  }
}

// 16 MFMAs of one sub-step.  sa/sb hold the scale words of the lane's rows shifted by
// 8 * (lane / 32), so byte 2 (SUB % 2) is the scale of the lane's K block.
template <int SUB>
__device__ __forceinline__ void gemm_mma(const GemmFrags& f, const uint32_t sa[4], const uint32_t sb[4],
                                         v16f_t acc[4][4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(f.a[i], f.b[j], acc[i][j], 4, 4, 2 * (SUB & 1),
                                                                  (int)sa[i], 2 * (SUB & 1), (int)sb[j]);
}

// Scheduling groups: one MFMA, then up to V global loads and D LDS reads, N times.
template <int N, int V, int D>
__device__ __forceinline__ void interleave() {
#pragma unroll
  for (int g = 0; g < N; ++g) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    if constexpr (V > 0) __builtin_amdgcn_sched_group_barrier(0x020, V, 0);
    if constexpr (D > 0) __builtin_amdgcn_sched_group_barrier(0x100, D, 0);
  }
}

template <bool BF16OUT, bool AMAX>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void k_gemm_mxfp4(
    const uint8_t* __restrict__ ac, const uint8_t* __restrict__ as, const uint8_t* __restrict__ bc,
    const uint8_t* __restrict__ bs, int M, int N, int K, int tiles_m, int tiles_n, void* __restrict__ cout,
    uint32_t* __restrict__ amax) {
  __shared__ GemmLds lds_;
  GemmStage* st = lds_.st;
  GemmScales* sc = lds_.sc;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  int tm, tn;
  gemm_tile(blockIdx.x, tiles_m, tiles_n, tm, tn);
  const int m0 = tm * kGemmTile, n0 = tn * kGemmTile;
  const int64_t ldq = K / 2, lds = K / 32;   // row strides of codes and scales, bytes
  const int nb = K / 128;                     // 128-element halves of a step
  const int nk = (nb + 1) / 2;                // steps; with nb odd the last one is half
  const int last_chunk_byte = (int)ldq - 16;  // last 16 bytes of a row of codes

  // Loader: chunk p = 256 j + tid of a stage is row 32 j + tid / 8, position tid % 8,
  // which holds global chunk (tid % 8) ^ gemm_swz(row) (gemm_swz depends on row % 16 =
  // (tid / 8) % 16 only).  Rows past the matrix read its last row (their products land
  // in C rows or columns that are not stored); chunks past k, in a half last step, read
  // the row's last 16 bytes (their MFMAs are skipped).
  const int lr = tid >> 3;
  const int gch = (tid & 7) ^ (int)gemm_swz((uint32_t)lr);
  // Row group j starts at the uniform row min(m0 + 32 j, M - 1) (scalar base); the
  // lane adds the 32-bit offset of its own (clamped) row, < 32 rows of ldq bytes.
  uint32_t oa[8], ob[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    oa[j] = (uint32_t)((min(m0 + 32 * j + lr, M - 1) - min(m0 + 32 * j, M - 1)) * (int)ldq);
    ob[j] = (uint32_t)((min(n0 + 32 * j + lr, N - 1) - min(n0 + 32 * j, N - 1)) * (int)ldq);
  }
  // Scale slice j of a chunk: this lane fetches row 64 j + 16 wave + lane/4, position
  // lane % 4, i.e. row word 4C + ((lane % 4) ^ scale_swz(row)), clamped to the row's
  // last word so that a partial last chunk stays inside the row.
  const int srow = 16 * wave + (lane >> 2);                      // row within the slice, + 64 j
  const int sd = (lane & 3) ^ (int)scale_swz((uint32_t)srow);    // the same for every j
  auto issue_scales = [&](int chunk, int j) {
    GemmScales& c = sc[chunk % 3];
    const int word = min(4 * chunk + sd, nb - 1);
    const int r = 64 * j + srow;
    __builtin_amdgcn_global_load_lds(as + (int64_t)min(m0 + r, M - 1) * lds + 4 * word,
                                     &c.a[(64 * j + 16 * wave) * 4], 4, 0, 0);
    __builtin_amdgcn_global_load_lds(bs + (int64_t)min(n0 + r, N - 1) * lds + 4 * word,
                                     &c.b[(64 * j + 16 * wave) * 4], 4, 0, 0);
  };
  auto issue = [&](int ks) {
    GemmStage& s = st[ks % kGemmStages];
    const uint32_t off = (uint32_t)min(ks * 128 + gch * 16, last_chunk_byte);
#pragma unroll
    for (int j = 0; j < 8; ++j)
      __builtin_amdgcn_global_load_lds(ac + (int64_t)min(m0 + 32 * j, M - 1) * ldq + (oa[j] + off),
                                       &s.a[j * 256 + wave * 64], 16, 0, 0);
#pragma unroll
    for (int j = 0; j < 8; ++j)
      __builtin_amdgcn_global_load_lds(bc + (int64_t)min(n0 + 32 * j, N - 1) * ldq + (ob[j] + off),
                                       &s.b[j * 256 + wave * 64], 16, 0, 0);
    issue_scales((ks >> 1) + 1, 2 * (ks & 1));
    issue_scales((ks >> 1) + 1, 2 * (ks & 1) + 1);
  };

  // Fragment reads for sub-step u: row wm*128 + 32 i + fr, chunk (2u + fh) ^ gemm_swz(fr).
  const int wm = wave & 1, wn = wave >> 1;
  const int fr = lane & 31, fh = lane >> 5;
  const uint32_t sw = gemm_swz((uint32_t)fr);
  const uint32_t rowA = (uint32_t)(wm * 128 + fr) * 128, rowB = (uint32_t)(wn * 128 + fr) * 128;
  uint32_t pos[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) pos[u] = (((uint32_t)(2 * u + fh)) ^ sw) * 16;

  // Scale words of step ks for the lane's rows (wm*128 + 32 i + fr for A, likewise B):
  // word 2 (ks % 2) + h (h = 0 for sub-steps 0-1, 1 for 2-3) at position ^ scale_swz(row),
  // which depends only on fr for these rows.
  const uint32_t fsw = scale_swz((uint32_t)fr);
  const uint32_t posA = (uint32_t)(wm * 128 + fr) * 4, posB = (uint32_t)(wn * 128 + fr) * 4;
  auto scales_of = [&](int ks, uint32_t sa_[2][4], uint32_t sb_[2][4]) {
    const GemmScales& c = sc[(ks >> 1) % 3];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint32_t d = ((uint32_t)(2 * (ks & 1) + h)) ^ fsw;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        sa_[h][i] = c.a[posA + d + 32 * 4 * i] >> (8 * fh);
        sb_[h][i] = c.b[posB + d + 32 * 4 * i] >> (8 * fh);
      }
    }
  };

  v16f_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = v16f_t{};

  // Pipeline: while the 16 MFMAs of one sub-step run, the fragments of the next are
  // read.  The barrier that publishes step ks+1 sits before the last sub-step of step
  // ks, after every fragment of step ks is in registers; right after it the loads of
  // step ks+2 go into the stage step ks used, so one step is in flight behind the one
  // being consumed.  With one wave per SIMD the matrix core idles whenever the wave
  // issues anything else between two MFMAs for longer than one MFMA lasts, so reads
  // and loads are interleaved one by one with the MFMAs (scheduling groups).
  // Every step runs the same body: the last two issue loads past k at clamped, in-bounds
  // addresses and read a stage nobody fills with data that is never used, which keeps
  // the accumulators out of joins that made the compiler shuffle and spill them.  With
  // k % 256 == 128 the last step has two sub-steps: the other two take zero codes.
#pragma unroll
  for (int j = 0; j < 4; ++j) issue_scales(0, j);
  issue(0);
  issue(1);
  wait_vm<kLoadsPerStep>();
  gemm_barrier();
  GemmFrags f0, f1;
  uint32_t sa[2][4], sb[2][4];
  gemm_read(st[0], rowA + pos[0], rowB + pos[0], f0);
  scales_of(0, sa, sb);
  const int half_step = (nb & 1) ? nk - 1 : -1;

  for (int ks = 0; ks < nk; ++ks) {
    const GemmStage& s = st[ks % kGemmStages];
    gemm_read(s, rowA + pos[1], rowB + pos[1], f1);
    gemm_mma<0>(f0, sa[0], sb[0], acc);
    interleave<8, 0, 1>();
    interleave<8, 0, 0>();
    __builtin_amdgcn_sched_barrier(0);
    gemm_read(s, rowA + pos[2], rowB + pos[2], f0);
    gemm_mma<1>(f1, sa[0], sb[0], acc);
    interleave<8, 0, 1>();
    interleave<8, 0, 0>();
    __builtin_amdgcn_sched_barrier(0);
    gemm_read(s, rowA + pos[3], rowB + pos[3], f1);
    {
      const int keep = ks == half_step ? 0 : -1;   // uniform; an AND, not a branch
#pragma unroll
      for (int i = 0; i < 4; ++i) f0.a[i] &= keep, f1.a[i] &= keep;
    }
    gemm_mma<2>(f0, sa[1], sb[1], acc);
    interleave<8, 0, 1>();
    interleave<8, 0, 0>();
    __builtin_amdgcn_sched_barrier(0);
    uint32_t sa1[4], sb1[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) sa1[i] = sa[1][i], sb1[i] = sb[1][i];
    wait_vm<0>();      // step ks+1 has landed (no later step has been issued yet)
    gemm_barrier();
    issue(ks + 2);
    scales_of(ks + 1, sa, sb);
    gemm_read(st[(ks + 1) % kGemmStages], rowA + pos[0], rowB + pos[0], f0);
    gemm_mma<3>(f1, sa1, sb1, acc);
    interleave<10, 2, 1>();
    interleave<6, 0, 1>();
    __builtin_amdgcn_sched_barrier(0);
  }
  wait_vm<0>();   // the loads issued past k land in LDS before anything reuses it

  // Epilogue: register q of block (i, j) is C row m0 + wm*128 + 32 i + 8(q/4) + 4 fh + q%4,
  // column n0 + wn*128 + 32 j + fr.
  if constexpr (BF16OUT) {
    // The 128 x 128 bf16 block goes through LDS, row-major, so that a store writes 16
    // bytes and four whole 256-byte rows per instruction (the registers hold one column
    // per lane, which would write half cache lines).  Each wave uses its own 32 KB once
    // every wave has finished reading the stages; pieces that cross the edge of C, or
    // rows not 16-byte aligned (n % 8 != 0), are stored element by element.
    gemm_barrier();
    const int br = m0 + wm * 128, bc0 = n0 + wn * 128;
    uint16_t* e = reinterpret_cast<uint16_t*>(&lds_) + wave * 128 * 128;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
#pragma unroll
        for (int q = 0; q < 16; ++q)
          e[(32 * i + 8 * (q >> 2) + 4 * fh + (q & 3)) * 128 + 32 * j + fr] = bf16_rne(acc[i][j][q]);
        __builtin_amdgcn_sched_barrier(0);   // one block at a time keeps few values live
      }
    uint16_t* c16 = static_cast<uint16_t*>(cout);
    const bool vec = (N & 7) == 0;
    uint32_t am = 0;   // largest stored bf16 magnitude
    for (int it = 0; it < 32; ++it) {
      const int row = 4 * it + (lane >> 4), c8 = (lane & 15) * 8;
      if (br + row >= M) continue;
      uint16_t* dst = c16 + (int64_t)(br + row) * N + bc0 + c8;
      const uint16_t* src = e + row * 128 + c8;
      if (vec && bc0 + c8 + 8 <= N) {
        const u32x4_g v = *reinterpret_cast<const u32x4_g*>(src);
        *reinterpret_cast<u32x4_g*>(dst) = v;
        if constexpr (AMAX)
          am = max(am, max(max(bf16x2_absmax(v[0]), bf16x2_absmax(v[1])), max(bf16x2_absmax(v[2]), bf16x2_absmax(v[3]))));
      } else {
        for (int x = 0; x < 8 && bc0 + c8 + x < N; ++x) {
          dst[x] = src[x];
          if constexpr (AMAX) am = max(am, (uint32_t)(src[x] & 0x7FFFu));
        }
      }
    }
    if constexpr (AMAX) post_amax(am << 16, amax);
    return;
  }
  uint32_t am = 0;   // largest stored fp32 magnitude
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int col = n0 + wn * 128 + 32 * j + fr;
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int row = m0 + wm * 128 + 32 * i + 8 * (q >> 2) + 4 * fh + (q & 3);
        if (row < M && col < N) {
          static_cast<float*>(cout)[(int64_t)row * N + col] = acc[i][j][q];
          if constexpr (AMAX) am = max(am, __float_as_uint(acc[i][j][q]) & 0x7FFFFFFFu);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  if constexpr (AMAX) post_amax(am, amax);
}

// ---------------------------------------------------------------------------------------
// NVFP4 1x16 operands: the scaled MFMA takes only power-of-two (E8M0) block scales, and an
// E4M3 scale has a 3-bit significand, so each element is decoded to r * s (at most six
// significant bits: exact in f16 and in bf16) and multiplied on a 16-bit MFMA with fp32
// accumulation, f16 (v_mfma_f32_32x32x16_f16) for NVFP4 operands and bf16 where an IF4
// operand takes part; the tensor scales are applied once to the fp32 sums.
// The scaled FP4 convert applies only the exponent of its scale operand (checked on the
// box with non-power-of-two scales), so the decode converts with scale 1 and multiplies
// by s afterwards.
// ---------------------------------------------------------------------------------------

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float v2f_t __attribute__((ext_vector_type(2)));

constexpr int kNvStages = 4;
constexpr int kNvLoads = 12;   // per wave and K step: 4 + 4 code chunks, 4 scale pieces

// A K step is 128 elements: 64 bytes of codes and 8 scale bytes per row.
struct NvStage {
  u32x4_g a[kGemmTile * 4];   // 256 rows x four 16-byte chunks (swizzled)
  u32x4_g b[kGemmTile * 4];
  uint32_t sa[kGemmTile * 2]; // the row's two scale words of the step
  uint32_t sb[kGemmTile * 2];
};

// Chunk c of staged row r at position c ^ nv_swz(r): 16 consecutive rows at one chunk
// fall in distinct bank groups with 32 or 64 banks.
__device__ __forceinline__ uint32_t nv_swz(uint32_t r) { return ((r >> 2) & 1u) | ((((r >> 1) ^ (r >> 3)) & 1u) << 1); }

// Eight E2M1 codes (one word, element 2i in the low nibble of byte i) times the block
// scale s -> eight bf16 in element order.  r * s is exact in fp32 and in bf16, so taking
// the high half of each fp32 is exact.
__device__ __forceinline__ uint32_t nv_pair(v2f_t p, float s) {
  return __builtin_amdgcn_perm(__float_as_uint(p.y * s), __float_as_uint(p.x * s), 0x07060302u);
}
__device__ __forceinline__ bf16x8_t nv_decode(uint32_t w, float s) {
  const uint32_t o0 = nv_pair(__builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 0), s);
  const uint32_t o1 = nv_pair(__builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 1), s);
  const uint32_t o2 = nv_pair(__builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 2), s);
  const uint32_t o3 = nv_pair(__builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 3), s);
  return __builtin_bit_cast(bf16x8_t, u32x4_g{o0, o1, o2, o3});
}

// The same decode to f16 for the f16 MFMA: r * s lies between 2^-10 and 2688 in magnitude
// (E2M1 magnitudes 0.5..6 times E4M3 scales 2^-9..448) with at most six significant bits,
// so it is exact in f16's normal range and the packed f16 multiply never rounds; the convert
// gives r itself (scale 1) and s is an exact f16 too.  Half the instructions of the bf16
// decode: one convert and one packed multiply per two elements.
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ f16x8_t nv_decode_h(uint32_t w, _Float16 s) {
  const f16x2_t ss = {s, s};
  const f16x2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0) * ss;
  const f16x2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1) * ss;
  const f16x2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2) * ss;
  const f16x2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3) * ss;
  return f16x8_t{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

__device__ __forceinline__ float e4m3_byte(uint32_t w, int byte) {
  switch (byte) {
    case 0: return __builtin_amdgcn_cvt_f32_fp8((int)w, 0);
    case 1: return __builtin_amdgcn_cvt_f32_fp8((int)w, 1);
    case 2: return __builtin_amdgcn_cvt_f32_fp8((int)w, 2);
    default: return __builtin_amdgcn_cvt_f32_fp8((int)w, 3);
  }
}

// IF4 operands [IF "2. 提案手法：IF4"]: a block whose scale byte has bit 7 set holds
// two's-complement INT4 codes q, restored as fl(q fl(6/7)), times the E4M3 scale of the
// byte's low seven bits.  Such an element e = fl(fl(q fl(6/7)) s) has up to 24
// significant bits, more than bf16 holds, so the MFMA takes it in two parts, hi = bf16(e)
// and lo = bf16(e - hi) (e - hi is exact in fp32), and the kernel issues a second MFMA
// with the lo parts: hi + lo is within (2^-16 + 2^-24) |e| of the restore times s (two
// bf16 roundings of at most 2^-8 each, after e's fp32 rounding), and every product of
// parts is exact in fp32.  E2M1 blocks of an IF4 operand decode exactly as above with
// lo = 0.  With both operands IF4 the lo x lo products (at most about 2^-16 of the
// product) are left out.
constexpr float kSixSevenths = 6.0f / 7.0f;   // fl(6/7)

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// Two fp32 values to packed bf16, rounded to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pk_bf16(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((v2f_t{a, b}), bf16x2_t));
}

// Eight elements of an IF4 operand (code word w, scale byte sb) as hi and lo bf16 parts.
__device__ __forceinline__ void if4_decode(uint32_t w, uint32_t sb, bf16x8_t& hi, bf16x8_t& lo) {
  const float s = __builtin_amdgcn_cvt_f32_fp8((int)(sb & 0x7Fu), 0);
  if (!(sb & 0x80u)) {
    hi = nv_decode(w, s);
    lo = __builtin_bit_cast(bf16x8_t, u32x4_g{0u, 0u, 0u, 0u});
    return;
  }
  uint32_t h[4], l[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int q0 = (int)(w << (28 - 8 * k)) >> 28, q1 = (int)(w << (24 - 8 * k)) >> 28;   // elements 2k, 2k+1
    const float v0 = ((float)q0 * kSixSevenths) * s, v1 = ((float)q1 * kSixSevenths) * s;
    h[k] = pk_bf16(v0, v1);
    l[k] = pk_bf16(v0 - __uint_as_float(h[k] << 16), v1 - __uint_as_float(h[k] & 0xFFFF0000u));
  }
  hi = __builtin_bit_cast(bf16x8_t, u32x4_g{h[0], h[1], h[2], h[3]});
  lo = __builtin_bit_cast(bf16x8_t, u32x4_g{l[0], l[1], l[2], l[3]});
}

// C = (A B^T) / (gs_a gs_b).  v_mfma_f32_32x32x16_f16 / _bf16 take, per lane, eight
// consecutive K elements of row l % 32 in its half l / 32 of the instruction's 16; K
// order inside a step is free as long as A and B agree, so MFMA q (0..7) of a step
// gives lane half 0 the row's code word q (elements 8q..8q+7, block q/2) and half 1 the
// word 8 + q (block 4 + q/2): a lane reads 32 contiguous bytes of codes and one scale
// word (blocks 4 fh .. 4 fh + 3) per row and step.
// IF4 bit 0 / bit 1: A / B is an IF4 operand.
template <bool BF16OUT, bool AMAX, int IF4>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void k_gemm_nvfp4(
    const uint8_t* __restrict__ ac, const uint8_t* __restrict__ as, const float* __restrict__ gsa,
    const uint8_t* __restrict__ bc, const uint8_t* __restrict__ bs, const float* __restrict__ gsb, int M, int N,
    int K, int tiles_m, int tiles_n, void* __restrict__ cout, uint32_t* __restrict__ amax, int tile_a, int tile_b) {
  __shared__ NvStage st[kNvStages];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  int tm, tn;
  gemm_tile(blockIdx.x, tiles_m, tiles_n, tm, tn);
  const int m0 = tm * kGemmTile, n0 = tn * kGemmTile;
  const int64_t ldq = K / 2, lds = K / 16;   // row strides of codes and scales, bytes
  const int nk = K / 128;

  // Codes: chunk p = 256 j + tid of a stage is row 64 j + tid / 4, position tid % 4,
  // holding global chunk (tid % 4) ^ nv_swz(row).  Rows past the matrix read its last
  // row; steps past k (issued by the last iterations) read the last step.
  const int lr = tid >> 2;
  const int gch = (tid & 3) ^ (int)nv_swz((uint32_t)lr);
  uint32_t oa[4], ob[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    oa[j] = (uint32_t)((min(m0 + 64 * j + lr, M - 1) - min(m0 + 64 * j, M - 1)) * (int)ldq);
    ob[j] = (uint32_t)((min(n0 + 64 * j + lr, N - 1) - min(n0 + 64 * j, N - 1)) * (int)ldq);
  }
  // Scales: piece g (0..7) of an operand is rows 32 g .. 32 g + 31, two words each;
  // wave w loads pieces 2w and 2w+1 of A and of B.  An operand with 16x16 scale tiles
  // (tile_a / tile_b = 4) reads the scale row of its row's tile, row / 16.
  auto issue = [&](int ks) {
    NvStage& s = st[ks % kNvStages];
    const int kc = min(ks, nk - 1);
    const uint32_t off = (uint32_t)(kc * 64 + gch * 16);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      __builtin_amdgcn_global_load_lds(ac + (int64_t)min(m0 + 64 * j, M - 1) * ldq + (oa[j] + off),
                                       &s.a[j * 256 + wave * 64], 16, 0, 0);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      __builtin_amdgcn_global_load_lds(bc + (int64_t)min(n0 + 64 * j, N - 1) * ldq + (ob[j] + off),
                                       &s.b[j * 256 + wave * 64], 16, 0, 0);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int g = 2 * wave + h, row = 32 * g + (lane >> 1);
      const int64_t so = (int64_t)kc * 8 + 4 * (lane & 1);
      __builtin_amdgcn_global_load_lds(as + (int64_t)(min(m0 + row, M - 1) >> tile_a) * lds + so, &s.sa[64 * g], 4,
                                       0, 0);
      __builtin_amdgcn_global_load_lds(bs + (int64_t)(min(n0 + row, N - 1) >> tile_b) * lds + so, &s.sb[64 * g], 4,
                                       0, 0);
    }
  };

  const int wm = wave & 1, wn = wave >> 1;
  const int fr = lane & 31, fh = lane >> 5;
  const uint32_t sw = nv_swz((uint32_t)fr);
  const uint32_t rowA = (uint32_t)(wm * 128 + fr) * 64, rowB = (uint32_t)(wn * 128 + fr) * 64;
  const uint32_t p0 = (((uint32_t)(2 * fh)) ^ sw) * 16, p1 = (((uint32_t)(2 * fh + 1)) ^ sw) * 16;
  const int srA = (wm * 128 + fr) * 2 + fh, srB = (wn * 128 + fr) * 2 + fh;

  v16f_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = v16f_t{};

  // Every step runs the same body (loads past k are clamped and never read), so the
  // wait count is the same everywhere: step ks has landed once at most the loads of
  // steps ks+1 and ks+2 remain.
  issue(0);
  issue(1);
  issue(2);
  for (int ks = 0; ks < nk; ++ks) {
    wait_vm<2 * kNvLoads>();
    gemm_barrier();   // step ks is in LDS for every wave; step ks-1's stage is free
    issue(ks + 3);
    const NvStage& s = st[ks % kNvStages];
    u32x4_g ra[4][2], rb[4][2];
    uint32_t wa[4], wb[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const char* pa = reinterpret_cast<const char*>(s.a) + rowA + i * 32 * 64;
      const char* pb = reinterpret_cast<const char*>(s.b) + rowB + i * 32 * 64;
      ra[i][0] = *reinterpret_cast<const u32x4_g*>(pa + p0);
      ra[i][1] = *reinterpret_cast<const u32x4_g*>(pa + p1);
      rb[i][0] = *reinterpret_cast<const u32x4_g*>(pb + p0);
      rb[i][1] = *reinterpret_cast<const u32x4_g*>(pb + p1);
      wa[i] = s.sa[srA + 64 * i];
      wb[i] = s.sb[srB + 64 * i];
    }
    // the scale bytes as f16 pairs, two per convert (E4M3 values are exact in f16)
    f16x2_t sha[4][2], shb[4][2];
    if constexpr (IF4 == 0) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        sha[i][0] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(wa[i], 1.0f, false);
        sha[i][1] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(wa[i], 1.0f, true);
        shb[i][0] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(wb[i], 1.0f, false);
        shb[i][1] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(wb[i], 1.0f, true);
      }
    }
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      if constexpr (IF4 == 0) {
        f16x8_t fa[4], fb[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          fa[i] = nv_decode_h(ra[i][q >> 2][q & 3], sha[i][q >> 2][(q >> 1) & 1]);
          fb[i] = nv_decode_h(rb[i][q >> 2][q & 3], shb[i][q >> 2][(q >> 1) & 1]);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(fa[i], fb[j], acc[i][j], 0, 0, 0);
      } else {
        // B's four fragments (and their lo parts) first, then A one fragment at a time, so
        // that only one A lo part is live: hi x hi, hi(A) x lo(B), lo(A) x hi(B).
        bf16x8_t fb[4], fbl[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if constexpr (IF4 & 2) if4_decode(rb[j][q >> 2][q & 3], (wb[j] >> (8 * (q >> 1))) & 0xFFu, fb[j], fbl[j]);
          else fb[j] = nv_decode(rb[j][q >> 2][q & 3], e4m3_byte(wb[j], q >> 1));
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          bf16x8_t fa, fal;
          if constexpr (IF4 & 1) if4_decode(ra[i][q >> 2][q & 3], (wa[i] >> (8 * (q >> 1))) & 0xFFu, fa, fal);
          else fa = nv_decode(ra[i][q >> 2][q & 3], e4m3_byte(wa[i], q >> 1));
#pragma unroll
          for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa, fb[j], acc[i][j], 0, 0, 0);
          if constexpr (IF4 & 2) {
#pragma unroll
            for (int j = 0; j < 4; ++j)
              acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa, fbl[j], acc[i][j], 0, 0, 0);
          }
          if constexpr (IF4 & 1) {
#pragma unroll
            for (int j = 0; j < 4; ++j)
              acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fal, fb[j], acc[i][j], 0, 0, 0);
          }
        }
      }
    }
  }
  wait_vm<0>();   // the loads issued past k land before anything reuses LDS

  // Tensor scales: C = sum / (gs_a gs_b), applied as one multiply by fl(1 / fl(gs_a gs_b)).
  const float inv = 1.0f / (gsa[0] * gsb[0]);
  if constexpr (BF16OUT) {
    gemm_barrier();
    const int br = m0 + wm * 128, bc0 = n0 + wn * 128;
    uint16_t* e = reinterpret_cast<uint16_t*>(&st[0]) + wave * 128 * 128;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
#pragma unroll
        for (int q = 0; q < 16; ++q)
          e[(32 * i + 8 * (q >> 2) + 4 * fh + (q & 3)) * 128 + 32 * j + fr] = bf16_rne(acc[i][j][q] * inv);
        __builtin_amdgcn_sched_barrier(0);
      }
    uint16_t* c16 = static_cast<uint16_t*>(cout);
    const bool vec = (N & 7) == 0;
    uint32_t am = 0;   // largest stored bf16 magnitude
    for (int it = 0; it < 32; ++it) {
      const int row = 4 * it + (lane >> 4), c8 = (lane & 15) * 8;
      if (br + row >= M) continue;
      uint16_t* dst = c16 + (int64_t)(br + row) * N + bc0 + c8;
      const uint16_t* src = e + row * 128 + c8;
      if (vec && bc0 + c8 + 8 <= N) {
        const u32x4_g v = *reinterpret_cast<const u32x4_g*>(src);
        *reinterpret_cast<u32x4_g*>(dst) = v;
        if constexpr (AMAX)
          am = max(am, max(max(bf16x2_absmax(v[0]), bf16x2_absmax(v[1])), max(bf16x2_absmax(v[2]), bf16x2_absmax(v[3]))));
      } else {
        for (int x = 0; x < 8 && bc0 + c8 + x < N; ++x) {
          dst[x] = src[x];
          if constexpr (AMAX) am = max(am, (uint32_t)(src[x] & 0x7FFFu));
        }
      }
    }
    if constexpr (AMAX) post_amax(am << 16, amax);
    return;
  }
  uint32_t am = 0;   // largest stored fp32 magnitude
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int col = n0 + wn * 128 + 32 * j + fr;
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int row = m0 + wm * 128 + 32 * i + 8 * (q >> 2) + 4 * fh + (q & 3);
        if (row < M && col < N) {
          const float v = acc[i][j][q] * inv;
          static_cast<float*>(cout)[(int64_t)row * N + col] = v;
          if constexpr (AMAX) am = max(am, __float_as_uint(v) & 0x7FFFFFFFu);
        }
      }
    }
  }
  if constexpr (AMAX) post_amax(am, amax);
}

}  // namespace

bool launch_gemm_mxfp4(const uint8_t* ac, const uint8_t* as, const uint8_t* bc, const uint8_t* bs, int64_t m,
                       int64_t n, int64_t k, bool bf16_out, void* c, float* amax, hipStream_t st) {
  const int tiles_m = (int)((m + kGemmTile - 1) / kGemmTile), tiles_n = (int)((n + kGemmTile - 1) / kGemmTile);
  const int64_t total = (int64_t)tiles_m * tiles_n;
  if (total > 0x7FFFFFFF) return false;
  uint32_t* ab = reinterpret_cast<uint32_t*>(amax);
  if (ab) k_gemm_amax_zero<<<1, 1, 0, st>>>(ab);
  // the amax fold only in the instances that report it: the others compile as without it
  auto kern = bf16_out ? (ab ? k_gemm_mxfp4<true, true> : k_gemm_mxfp4<true, false>)
                       : (ab ? k_gemm_mxfp4<false, true> : k_gemm_mxfp4<false, false>);
  kern<<<(unsigned)total, 256, 0, st>>>(ac, as, bc, bs, (int)m, (int)n, (int)k, tiles_m, tiles_n, c, ab);
  return true;
}

template <bool BF16OUT, bool AMAX>
static auto nvfp4_kernel(unsigned if4) {
  return if4 == 0 ? k_gemm_nvfp4<BF16OUT, AMAX, 0>
       : if4 == 1 ? k_gemm_nvfp4<BF16OUT, AMAX, 1>
       : if4 == 2 ? k_gemm_nvfp4<BF16OUT, AMAX, 2>
                  : k_gemm_nvfp4<BF16OUT, AMAX, 3>;
}

bool launch_gemm_nvfp4(const uint8_t* ac, const uint8_t* as, const float* gsa, const uint8_t* bc, const uint8_t* bs,
                       const float* gsb, int64_t m, int64_t n, int64_t k, bool bf16_out, void* c, float* amax,
                       unsigned flags, hipStream_t st) {
  const int tiles_m = (int)((m + kGemmTile - 1) / kGemmTile), tiles_n = (int)((n + kGemmTile - 1) / kGemmTile);
  const int64_t total = (int64_t)tiles_m * tiles_n;
  if (total > 0x7FFFFFFF) return false;
  uint32_t* ab = reinterpret_cast<uint32_t*>(amax);
  if (ab) k_gemm_amax_zero<<<1, 1, 0, st>>>(ab);
  const unsigned if4 = (flags >> 2) & 3u;
  auto kern = bf16_out ? (ab ? nvfp4_kernel<true, true>(if4) : nvfp4_kernel<true, false>(if4))
                       : (ab ? nvfp4_kernel<false, true>(if4) : nvfp4_kernel<false, false>(if4));
  kern<<<(unsigned)total, 256, 0, st>>>(ac, as, gsa, bc, bs, gsb, (int)m, (int)n, (int)k, tiles_m, tiles_n, c, ab,
                                        (flags & 1u) ? 4 : 0, (flags & 2u) ? 4 : 0);
  return true;
}

}  // namespace fp4q
