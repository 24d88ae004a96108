// fp4q_dev.hpp -- device-side building blocks of libfp4q (gfx950 / CDNA4).
//
// Element codec: E2M1 values (+-0, 0.5, 1, 1.5, 2, 3, 4, 6) as on
// qiita.com/nishiha/items/b98c2b931d588c4c81d5, section "NVFP4データの変換".  Block
// scales: E4M3 (max 448, section "NVFP4の表現できる最大値") and E8M0 (power of two,
// ultralytics.com/ja/glossary/fp4, section "FP4の仕組み").
//
// Arithmetic discipline: every quantity that decides a code is computed with the
// same IEEE binary32 roundings as the reference definition (no contraction; this
// file is compiled with -ffp-contract=off and uses fmaf only where stated).
#pragma once
#include "fp4q_internal.hpp"

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp4q {

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------------------
// bf16 / f32 loads
// ---------------------------------------------------------------------------

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Eight consecutive elements starting at element index `i` (16-byte aligned).
__device__ __forceinline__ void load8(const uint16_t* __restrict__ p, int64_t i, float out[8]) {
  uint4 w = *reinterpret_cast<const uint4*>(p + i);
  out[0] = bf16_lo(w.x); out[1] = bf16_hi(w.x);
  out[2] = bf16_lo(w.y); out[3] = bf16_hi(w.y);
  out[4] = bf16_lo(w.z); out[5] = bf16_hi(w.z);
  out[6] = bf16_lo(w.w); out[7] = bf16_hi(w.w);
}

__device__ __forceinline__ void load8(const float* __restrict__ p, int64_t i, float out[8]) {
  float4 a = *reinterpret_cast<const float4*>(p + i);
  float4 b = *reinterpret_cast<const float4*>(p + i + 4);
  out[0] = a.x; out[1] = a.y; out[2] = a.z; out[3] = a.w;
  out[4] = b.x; out[5] = b.y; out[6] = b.z; out[7] = b.w;
}

// Four consecutive elements, loaded non-temporally.  For kernels whose input is read
// once and whose load instructions each cover whole cache lines (k_nvfp4_2d,
// k_mxfp4): on fp32 8192 x 8192 the 16x16 quantizer runs 50.5 against 55.2 us with
// them.  Kernels whose instructions read parts of lines that later instructions
// complete are slower with non-temporal loads, since the parts no longer meet in L2.
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void load4(const float* __restrict__ p, float* o) {
  const f32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(p));
  o[0] = v.x; o[1] = v.y; o[2] = v.z; o[3] = v.w;
}
__device__ __forceinline__ void load4(const uint16_t* __restrict__ p, float* o) {
  const u32x2_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t*>(p));
  o[0] = bf16_lo(v.x); o[1] = bf16_hi(v.x); o[2] = bf16_lo(v.y); o[3] = bf16_hi(v.y);
}

// Sixteen consecutive elements per lane, where the 64 lanes of a wave take 64
// consecutive 16-element groups, read with whole cache lines per load instruction.
// stage_issue16 copies the wave's span (4 KB of fp32, 2 KB of bf16, starting at
// element e_wave) to the wave's LDS buffer `buf` by non-temporal direct loads
// (`global_load_lds_dwordx4`, no VGPR holds the data), each instruction covering 1 KB.
// Within an instruction lane j fetches the 16-byte chunk that reading lane j % G needs
// as its chunk j / G (G = 16 for fp32, 32 for bf16), so the chunks land transposed and
// the 16-byte LDS reads of 16 consecutive reading lanes fall on distinct banks.  Chunks
// at or past element n are fetched from the tensor's last chunk instead; only lanes
// whose groups lie past the end read them.  After stage_wait (every direct load of the
// wave done), stage_read16 gives each lane its 16 elements.  All lanes of the wave take
// part; each buffer is filled once.
__device__ __forceinline__ void lds_load16_nt(const void* g, uint32_t* lds) {
  __builtin_amdgcn_global_load_lds(g, lds, 16, 0, 2);   // aux bit 1: nt
}

template <typename T>
__device__ __forceinline__ void stage_issue16(const T* __restrict__ x, int64_t n, int64_t e_wave, uint32_t* buf) {
  constexpr int CH = 16 / (int)sizeof(T);          // elements per chunk: 4 (fp32) or 8 (bf16)
  constexpr int SPANS = (int)sizeof(T);            // 1 KB load instructions per wave
  constexpr int G = 64 / SPANS;                    // reading lanes per instruction
  const int lane = threadIdx.x & 63;
  const int c = lane / G, m = lane % G;            // fetch chunk c of reading lane m
#pragma unroll
  for (int sp = 0; sp < SPANS; ++sp) {
    int64_t e = e_wave + (int64_t)CH * (sp * 64 + (16 / CH) * m + c);
    e = e < n ? e : n - CH;
    lds_load16_nt(x + e, buf + sp * 256);
  }
}

__device__ __forceinline__ void stage_wait() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

template <typename T>
__device__ __forceinline__ void stage_read16(const uint32_t* buf, float out[16]) {
  constexpr int CH = 16 / (int)sizeof(T);
  constexpr int G = 64 / (int)sizeof(T);
  const int lane = threadIdx.x & 63;
  const int sp = lane / G, m = lane % G;
#pragma unroll
  for (int cc = 0; cc < 16 / CH; ++cc) {
    const u32x4_t w = *reinterpret_cast<const u32x4_t*>(buf + sp * 256 + 4 * (G * cc + m));
    if constexpr (sizeof(T) == 4) {
      out[4 * cc + 0] = __uint_as_float(w.x); out[4 * cc + 1] = __uint_as_float(w.y);
      out[4 * cc + 2] = __uint_as_float(w.z); out[4 * cc + 3] = __uint_as_float(w.w);
    } else {
      out[8 * cc + 0] = bf16_lo(w.x); out[8 * cc + 1] = bf16_hi(w.x);
      out[8 * cc + 2] = bf16_lo(w.y); out[8 * cc + 3] = bf16_hi(w.y);
      out[8 * cc + 4] = bf16_lo(w.z); out[8 * cc + 5] = bf16_hi(w.z);
      out[8 * cc + 6] = bf16_lo(w.w); out[8 * cc + 7] = bf16_hi(w.w);
    }
  }
}

// ---------------------------------------------------------------------------
// Division by a block scale in two operations, correctly rounded.
//
// For a divisor s > 0 with at most four significant bits (every E4M3 value, and 6)
// let zh be 1/s rounded toward zero and zl = fl(fl(1 - s*zh) * zh), which is >= 0.
// Then fl(t*zh + fl(t*zl)) -- one multiplication and one fused multiply-add -- is the
// correctly rounded quotient t/s for every binary32 t with a normal quotient: the
// repository's host check runs all 2^23 dividend significands against the eight
// divisor significands and spot-checks exponents.  Because zh and zl are both
// non-negative, both terms carry the dividend's sign and t = -0 gives -0.  A zero
// pair (zh = zl = 0) turns every dividend into a zero of its own sign, which is what
// a block whose scale rounded to zero needs.  The scheme is the one of Brisebarre,
// Muller and Raina for division by a constant known in advance (IEEE Trans. Comput.
// 53(8), 2004), with the high part rounded toward zero instead of to nearest.
// Quotients below the normal range may be off by an ulp; they are far below the
// smallest E2M1 rounding threshold, so no code depends on them.
// ---------------------------------------------------------------------------
struct RecipPair {
  float zh, zl;
};

__device__ __forceinline__ float div2(float t, RecipPair r) { return __builtin_fmaf(t, r.zh, t * r.zl); }

// The pair for an E4M3 value s > 0.  fl(1/s) comes from the hardware estimate
// (within 1 ulp) and one Newton step with an exact residual, which rounds correctly
// for every divisor with at most four significant bits (checked on the host for all
// 126 values with the estimate anywhere within 1 ulp).
__device__ __forceinline__ RecipPair recip_pair(float s) {
  const float r0 = __builtin_amdgcn_rcpf(s);
  float zh = __builtin_fmaf(__builtin_fmaf(-s, r0, 1.0f), r0, r0);
  float e = __builtin_fmaf(-s, zh, 1.0f);      // exact: 1 - s*zh needs few bits
  if (e < 0.0f) {                              // 1/s was rounded up: step one ulp down
    zh = __uint_as_float(__float_as_uint(zh) - 1u);
    e = __builtin_fmaf(-s, zh, 1.0f);
  }
  return RecipPair{zh, e * zh};
}

// Division by an arbitrary FP32 divisor y given rs = fl(1/y): q0 = fl(t*rs) is
// corrected once with the exact residual t - q0*y (Markstein).  Correct rounding is
// not guaranteed for every dividend, only for the dividend significands a caller has
// shown to be safe; the residual is written as -(q0*y - t) so zero dividends keep
// their sign.
__device__ __forceinline__ float div_rs(float t, float y, float rs) {
  const float q0 = t * rs;
  const float res = -__builtin_fmaf(q0, y, -t);
  return __builtin_fmaf(res, rs, q0);
}

// The pair for dividing by 6: zh = 0x3E2AAAAA (1/6 rounded down), 1 - 6*zh = 2^-24,
// zl = 2^-24 * zh.
__device__ __forceinline__ RecipPair recip6() {
  return RecipPair{__uint_as_float(0x3E2AAAAAu), __uint_as_float(0x322AAAAAu)};
}

// E4M3 code -> value via the hardware fp8 (OCP e4m3fn) convert; exact.
__device__ __forceinline__ float e4m3_decode(uint32_t code) {
  return __builtin_amdgcn_cvt_f32_fp8((int)code, 0);
}

// NVFP4 / IF4 block scale from the block max of |x*gs| (= fl(bamax*gs)):
// s = E4M3(fl(p / 6)), e4m3fn saturating at 448.  The hardware conversion rounds to
// nearest-even but does not saturate, so the value is clamped first.  The second
// converted value is +0, so the returned word is the scale byte itself.
__device__ __forceinline__ uint32_t nvfp4_scale_code(float p) {
  const float y = __builtin_fminf(div2(p, recip6()), 448.0f);
  // the convert writes bits 0..15 (y, then +0) and keeps bits 16..31 of its old operand:
  // any dead value does, and the mask lets uses that read 16 bits fold it away
  return __builtin_amdgcn_cvt_pk_fp8_f32(y, 0.0f, __float_as_uint(y), false) & 0xFFFFu;
}

// Reciprocal pairs of all 128 E4M3 codes, indexed by the code: a block divides by
// table[code].  Codes 0 (scale zero) and 0x7F (not a number; never produced, since
// scales saturate at 448) hold the zero pair.
struct RecipTable {
  RecipPair r[128];
};

// The pair for a scale byte (code 0: the zero pair).
__device__ __forceinline__ RecipPair recip_pair_code(uint32_t code) {
  const RecipPair r = recip_pair(e4m3_decode(code));
  const bool zero = code == 0u;
  return RecipPair{zero ? 0.0f : r.zh, zero ? 0.0f : r.zl};
}

// Fill by the first 128 threads of a workgroup; the caller synchronizes after.
__device__ __forceinline__ void fill_recip_table(RecipTable& tab) {
  const int c = threadIdx.x;
  if (c < 128) tab.r[c] = c == 0x7F ? RecipPair{0.0f, 0.0f} : recip_pair_code((uint32_t)c);
}

// ---------------------------------------------------------------------------
// E8M0 scale with round-to-nearest-even on the significand (MXFP4).
// y = fl(bamax/6).  Normal y: (bits + 0x3FFFFF + exponent_lsb) >> 23 rounds the
// significand to 0 bits, ties (significand exactly 1.5) to the even exponent code.
// Subnormal y (< 2^-126): nearest of {2^-127, 2^-126} with the same tie rule.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t e8m0_encode(float y) {
  uint32_t b = __float_as_uint(y);
  uint32_t code;
  if (b >= 0x00800000u) {
    code = (b + 0x3FFFFFu + ((b >> 23) & 1u)) >> 23;
  } else {
    code = b > 0x00600000u ? 1u : 0u;
  }
  return code > 254u ? 254u : code;
}

// ---------------------------------------------------------------------------
// E2M1 conversion on the gfx950 scaled converts.
// RTN: v_cvt_scalef32_pk_fp4_f32 rounds x / 2^exponent(scale) to nearest, ties to
// the even code, saturating at 6, sign copied; src0 lands in the low nibble.  With
// scale 1.0 it converts v itself.  `sel` picks the destination byte (others kept).
// ---------------------------------------------------------------------------
#define FP4Q_CVT_RTN(old, a, b, scale, sel) __builtin_amdgcn_cvt_scalef32_pk_fp4_f32((old), (a), (b), (scale), (sel))

// SR: the first element of v_cvt_scalef32_sr_pk_fp4_f32 rounds up iff
// frac + r/2^32 >= 1 on its E2M1 interval, where r is the 32-bit random operand, and the
// second element uses r << 1 (bit 31 dropped).  A 16-bit draw in the top half with the
// low half zero therefore gives exactly "up iff frac + r16/2^16 >= 1": the first element
// of a pair gets its draw as r = w & 0xFFFF0000 (the high half of a Philox word), the
// second as r = w << 15, so that r << 1 = w << 16 (the low half).  Each pair is
// converted twice from the same two values, keeping the first nibble of one result and
// the second of the other.  Only byte 0 of a result is defined: the builtin does not
// carry the old destination value through, so the other bytes are whatever the register
// held.
#define FP4Q_CVT_SR2(a, b, r32, scale) \
  __builtin_amdgcn_cvt_scalef32_sr_pk_fp4_f32(0u, f32x2{(a), (b)}, (r32), (scale), 0)

// ---------------------------------------------------------------------------
// Philox4x32-10 (Salmon et al., SC'11): multipliers 0xD2511F53 / 0xCD9E8D57,
// Weyl key increments 0x9E3779B9 / 0xBB67AE85, ten rounds.
// ---------------------------------------------------------------------------
struct U4 { uint32_t x, y, z, w; };

__device__ __forceinline__ U4 philox10(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3,
                                       uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    uint64_t p0 = (uint64_t)0xD2511F53u * c0;
    uint64_t p1 = (uint64_t)0xCD9E8D57u * c2;
    // three-input XOR in one instruction (truth table 0x96)
    uint32_t n0 = __builtin_amdgcn_bitop3_b32((uint32_t)(p1 >> 32), c1, k0, 0x96);
    uint32_t n2 = __builtin_amdgcn_bitop3_b32((uint32_t)(p0 >> 32), c3, k1, 0x96);
    c1 = (uint32_t)p1;
    c3 = (uint32_t)p0;
    c0 = n0;
    c2 = n2;
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
  return U4{c0, c1, c2, c3};
}

// Draws for the eight elements idx8*8 .. idx8*8+7 of SR stream `stream`: element e
// uses the high 16-bit half of word e >> 1 when e is even and the low half when e is
// odd, returned as the random operands the pair convert expects (see above).
__device__ __forceinline__ void sr_draws8(uint64_t idx8, uint32_t stream, uint32_t k0, uint32_t k1,
                                          uint32_t r32[8]) {
  U4 w = philox10((uint32_t)idx8, (uint32_t)(idx8 >> 32), stream, 0u, k0, k1);
  r32[0] = w.x & 0xFFFF0000u; r32[1] = w.x << 15;
  r32[2] = w.y & 0xFFFF0000u; r32[3] = w.y << 15;
  r32[4] = w.z & 0xFFFF0000u; r32[5] = w.z << 15;
  r32[6] = w.w & 0xFFFF0000u; r32[7] = w.w << 15;
}

// ---------------------------------------------------------------------------
// Encoders for 8 scaled values -> one 32-bit word of 8 nibbles (element k in
// bits 4k..4k+3).
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t pack8_rtn(const float v[8], float scale) {
  // The four converts overwrite all four bytes, so the starting value of the word is
  // irrelevant; starting from v[0]'s bits (dead after this) saves a register clear.
  uint32_t w = __float_as_uint(v[0]);
  w = FP4Q_CVT_RTN(w, v[0], v[1], scale, 0);
  w = FP4Q_CVT_RTN(w, v[2], v[3], scale, 1);
  w = FP4Q_CVT_RTN(w, v[4], v[5], scale, 2);
  w = FP4Q_CVT_RTN(w, v[6], v[7], scale, 3);
  return w;
}

__device__ __forceinline__ uint32_t pack8_sr(const float v[8], const uint32_t r32[8], float scale) {
  uint32_t t[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const uint32_t first = FP4Q_CVT_SR2(v[2 * k], v[2 * k + 1], r32[2 * k], scale);       // low nibble valid
    const uint32_t second = FP4Q_CVT_SR2(v[2 * k], v[2 * k + 1], r32[2 * k + 1], scale);  // high nibble valid
    t[k] = __builtin_amdgcn_bitop3_b32(first, second, 0x0F0F0F0Fu, 0xE4);   // (first & m) | (second & ~m)
  }
  const uint32_t u = __builtin_amdgcn_perm(t[1], t[0], 0x0C0C0400u);   // [t0.b0, t1.b0, 0, 0]
  const uint32_t w = __builtin_amdgcn_perm(t[3], t[2], 0x04000C0Cu);   // [0, 0, t2.b0, t3.b0]
  return u | w;
}

// ---------------------------------------------------------------------------
// FP6 elements (E2M3: FMT 0, E3M2: FMT 1), OCP MX formats with subnormals at exponent 0.
// ---------------------------------------------------------------------------
// Round to nearest, ties to the even code, saturating at code 31; the sign bit copied.
// Normal range: round the fp32 significand to MB bits by an integer add (ties to even)
// and re-bias the exponent; below the smallest normal 2^(1-BIAS) the step is
// 2^(1-BIAS-MB), reached by an exact power-of-two scaling and rint.  The two ranges meet:
// the subnormal result 2^MB is the smallest normal's code.
template <int FMT>
__device__ __forceinline__ uint32_t fp6_rtn(float v) {
  constexpr int MB = FMT ? 2 : 3, BIAS = FMT ? 3 : 1;
  constexpr float kMinNormal = FMT ? 0.25f : 1.0f;
  constexpr float kSubScale = (float)(1 << (BIAS - 1 + MB));
  const uint32_t u = __float_as_uint(v), au = u & 0x7FFFFFFFu;
  const float a = __uint_as_float(au);
  const uint32_t sub = (uint32_t)__builtin_rintf(a * kSubScale);
  const uint32_t nrm = ((au + ((1u << (22 - MB)) - 1u) + ((au >> (23 - MB)) & 1u)) >> (23 - MB)) -
                       ((uint32_t)(127 - BIAS) << MB);
  const uint32_t code = a < kMinNormal ? sub : nrm;
  return min(code, 31u) | ((u >> 31) << 5);
}

template <int FMT>
__device__ __forceinline__ float fp6_value(uint32_t c) {
  constexpr int MB = FMT ? 2 : 3, BIAS = FMT ? 3 : 1;
  const uint32_t e = (c >> MB) & ((1u << (5 - MB)) - 1u), m = c & ((1u << MB) - 1u);
  const float mag = e ? __uint_as_float(((e + 127u - BIAS) << 23) | (m << (23 - MB)))
                      : (float)m * (1.0f / (float)(1 << (BIAS - 1 + MB)));
  return (c & 0x20u) ? -mag : mag;
}

// The same rounding by gfx950's FP6 converts (v_cvt_scalef32_2xpk16_{fp6,bf6}_f32 with
// scale 1: nearest-even, saturating at the largest magnitude, sign copied, -0 and tiny
// negatives to the negative zero code), checked against the oracle's rounding on every
// grid point, midpoint and its neighbours, signed zeros, huge values and 13 000 random
// values in an in-bounds probe.  The instruction takes two 16-element vectors and writes
// 32 six-bit codes, code j at bits 6j of six words, code 2i from element i of the first
// vector and 2i + 1 from element i of the second; so the elements of two groups g and h
// (16 each) are handed over as (g0, g2, .., g14, h0, .., h14) and (g1, .., g15, h1, ..,
// h15), and g's codes land in words 0..2, h's in words 3..5.  The decode writes element j
// from code j.
typedef float f32x16v __attribute__((ext_vector_type(16)));
typedef float f32x32v __attribute__((ext_vector_type(32)));
typedef uint32_t u32x6v __attribute__((ext_vector_type(6)));

template <int FMT>
__device__ __forceinline__ u32x6v fp6_encode32(const float g[16], const float h[16]) {
  f32x16v a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = g[2 * i];
    b[i] = g[2 * i + 1];
    a[8 + i] = h[2 * i];
    b[8 + i] = h[2 * i + 1];
  }
  if constexpr (FMT == 0) return __builtin_amdgcn_cvt_scalef32_2xpk16_fp6_f32(a, b, 1.0f);
  else return __builtin_amdgcn_cvt_scalef32_2xpk16_bf6_f32(a, b, 1.0f);
}

template <int FMT>
__device__ __forceinline__ f32x32v fp6_decode32(u32x6v w) {
  if constexpr (FMT == 0) return __builtin_amdgcn_cvt_scalef32_pk32_f32_fp6(w, 1.0f);
  else return __builtin_amdgcn_cvt_scalef32_pk32_f32_bf6(w, 1.0f);
}

// 2^(k - 127) for an E8M0 code k: all of 2^-127 .. 2^127 are binary32 values.
__device__ __forceinline__ float e8m0_value(uint32_t k) { return k ? __uint_as_float(k << 23) : __uint_as_float(0x00400000u); }

// ---------------------------------------------------------------------------
// Cross-lane helpers (wave64).
// ---------------------------------------------------------------------------
// Maximum with the partner lane (lane ^ 1 or lane ^ 2 within each quad, by DPP) of a
// value that is >= 0: non-negative floats order like their bit patterns, so the
// comparison is an integer max (a float max would first canonicalize the moved value).
template <int XOR>
__device__ __forceinline__ float lane_xor_max(float v) {
  const int iv = __float_as_int(v);
  int other;
  if constexpr (XOR == 1)
    other = __builtin_amdgcn_mov_dpp(iv, 0xB1, 0xF, 0xF, false);   // [1,0,3,2]
  else
    other = __builtin_amdgcn_mov_dpp(iv, 0x4E, 0xF, 0xF, false);   // [2,3,0,1]
  return __uint_as_float(max((uint32_t)iv, (uint32_t)other));
}

// Workgroup barrier that orders LDS traffic only: unlike __syncthreads() it does not
// wait for outstanding global loads, so a prefetch of the next tile stays in flight.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

__device__ __forceinline__ float wave_max(float v) {
  for (int off = 32; off >= 1; off >>= 1) v = __builtin_fmaxf(v, __shfl_xor(v, off, 64));
  return v;
}

// Tensor encode scale gs = 2688 / amax (amax = 0 -> 1; overflow -> FLT_MAX),
// [qiita.com/nishiha/items/b98c2b931d588c4c81d5, "scaleの導出"]: the tensor's largest
// magnitude maps onto E4M3's 448 times the element format's block maximum (6 for E2M1;
// other block formats pass 448 * M).
__device__ __forceinline__ float tensor_scale_from_amax(float amax, float num = 2688.0f) {
  if (!(amax > 0.0f)) return 1.0f;
  float gs = __fdiv_rn(num, amax);
  return __builtin_fminf(gs, 3.40282347e38f);
}

__device__ __forceinline__ void atomic_max_nonneg(float* addr, float v) {
  // non-negative floats order like their bit patterns
  atomicMax(reinterpret_cast<unsigned int*>(addr), __float_as_uint(v));
}

// Where an amax pass posts its workgroup maxima, and where a quantizer finds the
// tensor amax: a float the call zeroed first (atomic max on its bits), or the
// two-pass state of a workspace (TwoPassAmax, with the protocol stated there).  Each
// workgroup posts once, from one thread.
__device__ __forceinline__ void post_amax(const AmaxSink& s, float m) {
  if (s.tp) {
    const uint32_t e = s.tp->ea;   // no workgroup of an amax pass writes it
    atomicMax(&s.tp->slot[e & 1u][0], __float_as_uint(m));
    if (blockIdx.x == 0) {
      s.tp->eq = e;                   // read by the quantizer that follows
      s.tp->slot[(e + 1u) & 1u][0] = 0u;   // the next call's slot; nobody reads it now
    }
  } else {
    atomic_max_nonneg(s.f, m);
  }
}

// The tensor scale from the source; workgroup 0's first thread publishes it (and the
// amax, when it came from a pass of this call) and hands the slot back.
__device__ __forceinline__ float tensor_scale_publish(const AmaxSource& s, float* tensor_scale,
                                                      float num = 2688.0f) {
  float a;
  uint32_t e = 0u;
  if (s.tp) {
    e = s.tp->eq;   // no workgroup of a quantizer writes it
    a = __uint_as_float(s.tp->slot[e & 1u][0]);
  } else {
    a = *s.f;
  }
  const float gs = tensor_scale_from_amax(a, num);
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    *tensor_scale = gs;
    if (s.out) *s.out = a;
    if (s.tp) s.tp->ea = e + 1u;   // the next call's amax pass posts into the other slot
  }
  return gs;
}

}  // namespace fp4q
