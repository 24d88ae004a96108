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
#include <type_traits>

#include "fp4q_internal.hpp"

namespace fp4q {
namespace {

typedef int v8i_t __attribute__((ext_vector_type(8)));
typedef float v16f_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_g __attribute__((ext_vector_type(4)));

constexpr int kGemmTile = 256;     // rows of A and of B per workgroup tile
constexpr int kGemmStages = 4;
constexpr int kLoadsPerStep = 10;  // global_load_lds per wave and K step: 4 + 4 code chunks, 2 scale slices

struct GemmStage {
  u32x4_g a[kGemmTile * 4];   // 256 rows x four 16-byte chunks (swizzled)
  u32x4_g b[kGemmTile * 4];
};

// Scales travel in chunks of four K steps: 16 bytes per row (row-major input keeps a
// row's scales for consecutive steps together, so one access per row brings four
// steps; a word per row and step would touch a cache line per row on every step).
// Three chunk buffers; the chunk for steps 4C..4C+3 is loaded in four slices of 64
// rows, one with each of the code loads of steps 4C-4 .. 4C-1, so every step issues
// the same number of loads.  Within a row, the word of step 4C+d sits at position
// d ^ scale_swz(row), spreading 32 consecutive rows over distinct banks.
struct GemmScales {
  uint32_t a[kGemmTile * 4];
  uint32_t b[kGemmTile * 4];
};
__device__ __forceinline__ uint32_t scale_swz(uint32_t r) { return (r >> 3) & 3u; }

struct GemmLds {
  GemmStage st[kGemmStages];
  GemmScales sc[3];
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
// The LDS wait goes through the builtin so that the compiler's own wait insertion knows
// every earlier LDS read is complete and adds no later wait for them.
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

// One 64-element K sub-step of a wave's 128 x 128 block: the 4 A and 4 B fragments.
struct GemmFrags {
  v8i_t a[4], b[4];
};

__device__ __forceinline__ void gemm_read(const GemmStage& s, uint32_t offA, uint32_t offB, GemmFrags& f) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const u32x4_g va = *reinterpret_cast<const u32x4_g*>(reinterpret_cast<const char*>(s.a) + offA + i * 32 * 64);
    const u32x4_g vb = *reinterpret_cast<const u32x4_g*>(reinterpret_cast<const char*>(s.b) + offB + i * 32 * 64);
    f.a[i] = v8i_t{(int)va.x, (int)va.y, (int)va.z, (int)va.w, 0, 0, 0, 0};
    f.b[i] = v8i_t{(int)vb.x, (int)vb.y, (int)vb.z, (int)vb.w, 0, 0, 0, 0};
  }
}

// The scale words of the lane's A and B rows, shifted so that byte 2 sub holds the
// scale of the lane's K block in sub-step sub (block 2 sub + fh of the step).
template <int SUB>
__device__ __forceinline__ void gemm_mma(const GemmFrags& f, const uint32_t sa[4], const uint32_t sb[4],
                                         v16f_t acc[4][4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(f.a[i], f.b[j], acc[i][j], 4, 4, 2 * SUB,
                                                                  (int)sa[i], 2 * SUB, (int)sb[j]);
}

template <bool BF16OUT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void k_gemm_mxfp4(
    const uint8_t* __restrict__ ac, const uint8_t* __restrict__ as, const uint8_t* __restrict__ bc,
    const uint8_t* __restrict__ bs, int M, int N, int K, int tiles_m, int tiles_n, void* __restrict__ cout) {
  __shared__ GemmLds lds_;
  GemmStage* st = lds_.st;
  GemmScales* sc = lds_.sc;
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
  // Scale slice j of a chunk: this lane fetches row 64 j + 16 wave + lane/4, position
  // lane % 4, i.e. the word of step 4C + (lane % 4) ^ scale_swz(row), clamped to the
  // last step so that a partial last chunk stays inside the row.
  const int srow = 16 * wave + (lane >> 2);   // row within the slice, + 64 j
  const int sd = (lane & 3) ^ (int)scale_swz((uint32_t)srow);   // the same for every j
  auto issue_scales = [&](int chunk, int j) {
    GemmScales& c = sc[chunk % 3];
    const int stp = min(4 * chunk + sd, nk - 1);
    const int r = 64 * j + srow;
    __builtin_amdgcn_global_load_lds(as + (int64_t)min(m0 + r, M - 1) * lds + 4 * stp, &c.a[(64 * j + 16 * wave) * 4],
                                     4, 0, 0);
    __builtin_amdgcn_global_load_lds(bs + (int64_t)min(n0 + r, N - 1) * lds + 4 * stp, &c.b[(64 * j + 16 * wave) * 4],
                                     4, 0, 0);
  };
  auto issue = [&](int ks) {
    GemmStage& s = st[ks % kGemmStages];
    const int64_t ko = (int64_t)ks * 64;
#pragma unroll
    for (int j = 0; j < 4; ++j) __builtin_amdgcn_global_load_lds(pa[j] + ko, &s.a[j * 256 + wave * 64], 16, 0, 0);
#pragma unroll
    for (int j = 0; j < 4; ++j) __builtin_amdgcn_global_load_lds(pb[j] + ko, &s.b[j * 256 + wave * 64], 16, 0, 0);
    issue_scales((ks >> 2) + 1, ks & 3);
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

  // Pipeline: while the 16 MFMAs of one sub-step run, the fragments of the next one
  // are already being read.  The barrier that publishes step ks+1 sits between the two
  // sub-steps of step ks, so the MFMAs never wait for it; right after it the loads of
  // step ks+3 go into the stage step ks-1 used (its last reads fed MFMAs issued before
  // the barrier), leaving two steps in flight behind the one being consumed.
  // The scale word of step ks for the lane's rows wm*128 + 32 i + fr (A) and
  // wn*128 + 32 i + fr (B): position ((ks & 3) ^ scale_swz(row)) of the row, and
  // scale_swz depends only on fr for these rows.
  const uint32_t fsw = scale_swz((uint32_t)fr);
  const uint32_t posA = (uint32_t)(wm * 128 + fr) * 4, posB = (uint32_t)(wn * 128 + fr) * 4;
  auto scales_of = [&](int ks, uint32_t sa_[4], uint32_t sb_[4]) {
    const GemmScales& c = sc[(ks >> 2) % 3];
    const uint32_t d = ((uint32_t)ks & 3u) ^ fsw;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      sa_[i] = c.a[posA + d + 32 * 4 * i] >> (8 * fh);
      sb_[i] = c.b[posB + d + 32 * 4 * i] >> (8 * fh);
    }
  };
#pragma unroll
  for (int j = 0; j < 4; ++j) issue_scales(0, j);
#pragma unroll
  for (int p = 0; p < kGemmStages - 1; ++p)
    if (p < nk) issue(p);
  if (nk >= 3) wait_vm<2 * kLoadsPerStep>();
  else if (nk == 2) wait_vm<kLoadsPerStep>();
  else wait_vm<0>();
  gemm_barrier();
  GemmFrags cur, nxt;
  uint32_t sa[4], sb[4];
  gemm_read(st[0], rowA + pos0, rowB + pos0, cur);
  scales_of(0, sa, sb);

  // One K step; MODE 0: steps ks+1 .. ks+3 exist (refill with ks+3), 3: ks+1 and ks+2
  // exist, 1: only ks+1, 2: ks is the last.  The body has no branch.  With one wave
  // per SIMD the matrix core idles whenever the wave issues anything else between two
  // MFMAs for longer than one MFMA lasts, so the reads and loads are interleaved one by
  // one with the MFMAs (scheduling groups); only the wait and the barrier stand alone.
  auto step = [&](int ks, auto mode) {
    constexpr int MODE = decltype(mode)::value;
    const GemmStage& s = st[ks % kGemmStages];
    gemm_read(s, rowA + pos1, rowB + pos1, nxt);
    gemm_mma<0>(cur, sa, sb, acc);
    uint32_t sa1[4], sb1[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) sa1[i] = sa[i], sb1[i] = sb[i];
#pragma unroll
    for (int g = 0; g < 8; ++g) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // one LDS read
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (MODE != 2) {
      // step ks+1 has landed once at most step ks+2's loads remain
      if constexpr (MODE == 0 || MODE == 3) wait_vm<kLoadsPerStep>();
      else wait_vm<0>();
      gemm_barrier();
      if constexpr (MODE == 0) issue(ks + 3);
      const GemmStage& s1 = st[(ks + 1) % kGemmStages];
      scales_of(ks + 1, sa, sb);
      gemm_read(s1, rowA + pos0, rowB + pos0, cur);
    }
    gemm_mma<1>(nxt, sa1, sb1, acc);
    if constexpr (MODE == 0) {
#pragma unroll
      for (int g = 0; g < 10; ++g) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);   // one global load
      }
#pragma unroll
      for (int g = 0; g < 6; ++g) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      }
    } else if constexpr (MODE != 2) {
#pragma unroll
      for (int g = 0; g < 12; ++g) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
  };
  int ks = 0;
  for (; ks + 3 < nk; ++ks) step(ks, std::integral_constant<int, 0>{});
  if (ks + 2 < nk) step(ks++, std::integral_constant<int, 3>{});
  if (ks + 1 < nk) step(ks++, std::integral_constant<int, 1>{});
  step(ks, std::integral_constant<int, 2>{});

  // Epilogue: register q of block (i, j) is C row m0 + wm*128 + 32 i + 8(q/4) + 4 fh + q%4,
  // column n0 + wn*128 + 32 j + fr.
  if constexpr (BF16OUT) {
    // The 128 x 128 bf16 block goes through LDS, row-major, so that a store writes 16
    // bytes and four whole 256-byte rows per instruction (the registers hold one column
    // per lane, which would write half cache lines).  Each wave uses its own 32 KB once
    // every wave has finished reading the stages; pieces that cross the edge of C, or
    // rows not 16-byte aligned (n % 8 != 0), are stored element by element.
    gemm_barrier();
    const int br = m0 + wm * 128, bc = n0 + wn * 128;
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
    for (int it = 0; it < 32; ++it) {
      const int row = 4 * it + (lane >> 4), c8 = (lane & 15) * 8;
      if (br + row >= M) continue;
      uint16_t* dst = c16 + (int64_t)(br + row) * N + bc + c8;
      const uint16_t* src = e + row * 128 + c8;
      if (vec && bc + c8 + 8 <= N) {
        *reinterpret_cast<u32x4_g*>(dst) = *reinterpret_cast<const u32x4_g*>(src);
      } else {
        for (int x = 0; x < 8 && bc + c8 + x < N; ++x) dst[x] = src[x];
      }
    }
    return;
  }
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
