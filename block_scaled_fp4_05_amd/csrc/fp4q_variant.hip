// fp4q_variant.hip -- block-format variants on NVFP4's two-level scaling, from the
// explainer of "Adaptive Block-Scaled Data Types" (gist.science/ja/paper/2603.28765):
//   Four Over Six (section "1. 背景と問題点"): the block maximum maps to 4 instead of 6,
//     so the E2M1 values +-6 are never produced;
//   NVINT4 (section "3. 主要な貢献", the INT4 baseline): INT4 elements, block max -> 7;
//   IF3 and IF6 (section "2. 提案手法：IF4", extensibility): per block the better of an FP
//     and an INT candidate, as IF4 does at 4 bits -- FP3 E2M0 (0, 1, 2, 4) against INT3,
//     and FP6 E2M3 (max 7.5) against INT6, the INT candidate scaled by the ratio of the
//     two formats' maxima and restored with its inverse; the choice is flagged in bit 7
//     of the block's E4M3 scale byte;
//   IF4 itself through the same code path (byte-identical to k_if4).
// Every variant: 16-element row blocks, gs = fl(448 M / amax), s = E4M3(fl(fl(bamax gs) / M)),
// v = fl(fl(x gs) / s); M is the format's block maximum.
#include "fp4q_dev.hpp"
#include "fp4q_internal.hpp"

namespace fp4q {

// Compile-time description of a variant.
template <int V> struct Var;
template <> struct Var<0> {   // Four Over Six
  static constexpr int kBits = 4, kQ = 0;
  static constexpr bool kFp = true, kInt = false, kDirect = false;
  static constexpr float kM = 4.0f, kC = 0.0f, kCinv = 0.0f;
};
template <> struct Var<1> {   // NVINT4
  static constexpr int kBits = 4, kQ = 7;
  static constexpr bool kFp = false, kInt = true, kDirect = true;
  static constexpr float kM = 7.0f, kC = 1.0f, kCinv = 1.0f;
};
template <> struct Var<2> {   // IF3: FP3 E2M0 or INT3
  static constexpr int kBits = 3, kQ = 3;
  static constexpr bool kFp = true, kInt = true, kDirect = false;
  static constexpr float kM = 4.0f, kC = 3.0f / 4.0f, kCinv = 4.0f / 3.0f;
};
template <> struct Var<3> {   // IF4: E2M1 or INT4 (the 6/7 rule)
  static constexpr int kBits = 4, kQ = 7;
  static constexpr bool kFp = true, kInt = true, kDirect = false;
  static constexpr float kM = 6.0f, kC = 7.0f / 6.0f, kCinv = 6.0f / 7.0f;
};
template <> struct Var<4> {   // IF6: FP6 E2M3 or INT6
  static constexpr int kBits = 6, kQ = 31;
  static constexpr bool kFp = true, kInt = true, kDirect = false;
  static constexpr float kM = 7.5f, kC = 31.0f / 7.5f, kCinv = 7.5f / 31.0f;
};

// fl(p / M), correctly rounded: M = 4 is an exact scaling, M = 6 the reciprocal pair,
// otherwise IEEE division (once per block).
template <int V>
__device__ __forceinline__ float div_block_max(float p) {
  if constexpr (Var<V>::kM == 4.0f) return p * 0.25f;
  else if constexpr (Var<V>::kM == 6.0f) return div2(p, recip6());
  else return __fdiv_rn(p, Var<V>::kM);
}

// E4M3 code of y >= 0, saturating at 448 (the convert rounds to nearest even).
__device__ __forceinline__ uint32_t e4m3_code(float y) {
  y = __builtin_fminf(y, 448.0f);
  return __builtin_amdgcn_cvt_pk_fp8_f32(y, 0.0f, __float_as_uint(y), false) & 0xFFu;
}

// FP3 E2M0 code of v: nearest of 0, 1, 2, 4 with ties to the even code (0.5 -> 0,
// 1.5 -> 2, 3 -> 2), saturating at 4; sign in bit 2.  Returns the code and its value.
__device__ __forceinline__ uint32_t fp3_rtn(float v, float& r) {
  const float a = __builtin_fabsf(v);
  const uint32_t c = (uint32_t)(a > 0.5f) + (uint32_t)(a >= 1.5f) + (uint32_t)(a > 3.0f);
  const float mag = c ? __uint_as_float((c + 126u) << 23) : 0.0f;   // 2^(c-1)
  const uint32_t neg = __float_as_uint(v) >> 31;
  r = neg ? -mag : mag;
  return c | (neg << 2);
}

// Sixteen codes of `bits` bits each, code k at bits bits*k of a little-endian word.
struct Codes16 {
  uint32_t w[3];
};

template <int BITS>
__device__ __forceinline__ void put16(Codes16& o, int k, uint32_t code) {
  const int b = BITS * k;
  o.w[b >> 5] |= code << (b & 31);
  if ((b & 31) + BITS > 32) o.w[(b >> 5) + 1] |= code >> (32 - (b & 31));
}

template <int BITS>
__device__ __forceinline__ uint32_t get16(const Codes16& o, int k) {
  const int b = BITS * k;
  uint32_t c = o.w[b >> 5] >> (b & 31);
  if ((b & 31) + BITS > 32) c |= o.w[(b >> 5) + 1] << (32 - (b & 31));
  return c & ((1u << BITS) - 1u);
}

constexpr int kVarBlocks = 4;   // blocks per lane, all loads issued first (as k_if4)

// Restore values of an INT candidate, fl((i - 2^(BITS-1)) * cinv) for i = 0 .. 2^BITS - 1,
// read at the address one shift-and-add makes of the rounded value's bits (as k_if4).
struct VarRestore {
  float r[64];
};
constexpr uint32_t kMagicBits = 0x4B400000u;   // bits of 1.5 * 2^23

// Whether the INT candidate needs its clamp with a normal block scale: the scale is at
// least 15/16 of fl(bamax gs)/M, so |v| <= M * 16/15 (one ulp more at most) and the
// clamp can only act if fl(v * c) may reach kQ + 1/2.
template <int V>
constexpr bool clamp_always() {
  using D = Var<V>;
  return D::kInt && (D::kM * 16.0f / 15.0f * (D::kDirect ? 1.0f : D::kC) * 1.0001f >= (float)D::kQ + 0.5f);
}

// One block: v holds x * gs on entry.  Writes the packed codes and the flagged scale.
template <int V, bool CLAMP>
__device__ __forceinline__ void variant_block(float (&v)[16], uint32_t sc, const RecipPair rp, const VarRestore& rt,
                                              Codes16& out, uint32_t& scale_byte) {
  using D = Var<V>;
  constexpr int BITS = D::kBits;
#pragma unroll
  for (int k = 0; k < 16; ++k) v[k] = div2(v[k], rp);

  Codes16 fc{{0u, 0u, 0u}}, ic{{0u, 0u, 0u}};
  float e_fp = 0.0f, e_int = 0.0f;
  if constexpr (D::kFp) {
    float rf[16];
    if constexpr (BITS == 4) {
      fc.w[0] = pack8_rtn(v, 1.0f);
      fc.w[1] = pack8_rtn(v + 8, 1.0f);
#define FP4Q_DEC(W, Q, O)                                                  \
  {                                                                        \
    const f32x2 d = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(W, 1.0f, Q); \
    rf[O + 2 * Q] = d[0];                                                  \
    rf[O + 2 * Q + 1] = d[1];                                              \
  }
      FP4Q_DEC(fc.w[0], 0, 0) FP4Q_DEC(fc.w[0], 1, 0) FP4Q_DEC(fc.w[0], 2, 0) FP4Q_DEC(fc.w[0], 3, 0)
      FP4Q_DEC(fc.w[1], 0, 8) FP4Q_DEC(fc.w[1], 1, 8) FP4Q_DEC(fc.w[1], 2, 8) FP4Q_DEC(fc.w[1], 3, 8)
#undef FP4Q_DEC
    } else if constexpr (BITS == 3) {
#pragma unroll
      for (int k = 0; k < 16; ++k) put16<3>(fc, k, fp3_rtn(v[k], rf[k]));
    } else {
      // FP6 E2M3 by the hardware convert and its decode (the block given twice)
      const u32x6v cw = fp6_encode32<0>(v, v);
      fc.w[0] = cw[0];
      fc.w[1] = cw[1];
      fc.w[2] = cw[2];
      const f32x32v d = fp6_decode32<0>(cw);
#pragma unroll
      for (int k = 0; k < 16; ++k) rf[k] = d[k];
    }
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const float d = v[k] - rf[k];
      e_fp = __builtin_fmaf(d, d, e_fp);
    }
  }
  if constexpr (D::kInt) {
    const float magic = 12582912.0f;   // 1.5 * 2^23: adding it rounds to an integer, ties to even
    // &rt.r[q + 2^(BITS-1)] = rt.r + (bits(y) - kMagicBits + 2^(BITS-1)), in 32-bit LDS addresses
    const float* base = rt.r + (1u << (BITS - 1)) - kMagicBits;
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      float w = D::kDirect ? v[k] : v[k] * D::kC;
      if constexpr (CLAMP) w = __builtin_amdgcn_fmed3f(w, -(float)D::kQ, (float)D::kQ);
      const float y = w + magic;
      const float ri = D::kDirect ? y - magic : base[__float_as_uint(y)];
      const float d = v[k] - ri;
      e_int = __builtin_fmaf(d, d, e_int);
      put16<BITS>(ic, k, __float_as_uint(y) & ((1u << BITS) - 1u));   // two's complement code
    }
  }
  const bool use_int = D::kInt && (!D::kFp || e_int < e_fp);
  out = use_int ? ic : fc;
  scale_byte = sc | (D::kFp && use_int ? 0x80u : 0u);
}

template <typename T, int V, bool CHECK>
__device__ __forceinline__ void variant_lane(const T* __restrict__ x, int64_t n16, float gs, const RecipTable& rtab,
                                             const VarRestore& rt, uint8_t* __restrict__ codes,
                                             uint8_t* __restrict__ scales) {
  using D = Var<V>;
  constexpr int BITS = D::kBits;
  const int64_t g0 = (int64_t)blockIdx.x * (256 * kVarBlocks) + threadIdx.x;
  float xv[kVarBlocks][16];
#pragma unroll
  for (int j = 0; j < kVarBlocks; ++j) {
    const int64_t g = CHECK ? min(g0 + 256 * j, n16 - 1) : g0 + 256 * j;   // past the end: reload, not stored
    load8(x, g * 16, xv[j]);
    load8(x, g * 16 + 8, xv[j] + 8);
  }
#pragma unroll
  for (int j = 0; j < kVarBlocks; ++j) {
    const int64_t g = g0 + 256 * j;
    float m = 0.0f;
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      xv[j][k] = xv[j][k] * gs;
      m = __builtin_fmaxf(m, __builtin_fabsf(xv[j][k]));
    }
    const uint32_t sc = e4m3_code(div_block_max<V>(m));
    const RecipPair rp = rtab.r[sc];
    Codes16 c;
    uint32_t sb;
    if constexpr (clamp_always<V>() || !D::kInt) {
      variant_block<V, D::kInt>(xv[j], sc, rp, rt, c, sb);
    } else {
      // the clamp only for waves holding a block whose scale is subnormal (uniform branch)
      if (__builtin_amdgcn_ballot_w64(sc < 8u) != 0) variant_block<V, true>(xv[j], sc, rp, rt, c, sb);
      else variant_block<V, false>(xv[j], sc, rp, rt, c, sb);
    }
    if (!CHECK || g < n16) {
      if constexpr (BITS == 4) {
        *reinterpret_cast<uint2*>(codes + g * 8) = make_uint2(c.w[0], c.w[1]);
      } else if constexpr (BITS == 3) {
        uint16_t* dst = reinterpret_cast<uint16_t*>(codes + g * 6);   // 2-byte aligned
        dst[0] = (uint16_t)c.w[0];
        dst[1] = (uint16_t)(c.w[0] >> 16);
        dst[2] = (uint16_t)c.w[1];
      } else {
        uint32_t* dst = reinterpret_cast<uint32_t*>(codes + g * 12);
        dst[0] = c.w[0];
        dst[1] = c.w[1];
        dst[2] = c.w[2];
      }
      scales[g] = (uint8_t)sb;
    }
  }
}

template <typename T, int V>
__global__ __launch_bounds__(256) void k_variant(const T* __restrict__ x, int64_t n16, AmaxSource amax,
                                                 float* __restrict__ tensor_scale, uint8_t* __restrict__ codes,
                                                 uint8_t* __restrict__ scales) {
  using D = Var<V>;
  __shared__ RecipTable rtab;
  __shared__ VarRestore rt;
  fill_recip_table(rtab);
  if (threadIdx.x < (1u << D::kBits))
    rt.r[threadIdx.x] = (float)((int)threadIdx.x - (1 << (D::kBits - 1))) * D::kCinv;
  __syncthreads();
  const float gs = tensor_scale_publish(amax, tensor_scale, 448.0f * D::kM);
  if ((int64_t)(blockIdx.x + 1) * (256 * kVarBlocks) <= n16)
    variant_lane<T, V, false>(x, n16, gs, rtab, rt, codes, scales);
  else
    variant_lane<T, V, true>(x, n16, gs, rtab, rt, codes, scales);
}

// x_hat = fl(fl(r * s) / gs) for the 3- and 6-bit formats (the 4-bit ones go through
// k_dequant).  As in k_dequant a lane takes 8 consecutive elements (half a block) per step
// and the lanes of a wave consecutive spans, so every store instruction writes one
// contiguous 1 KiB (bf16) or 2 KiB (fp32); the lane reads its block's packed codes and
// scale byte (the partner lane reads the same).  The division is the corrected
// reciprocal of k_dequant: correctly rounded for every dividend any of these formats
// forms (checked exhaustively on the host) while s/gs lies in [2^-98, 2^96]; IEEE
// division otherwise.  INT restores come from a table as in the quantizer.
template <int V, bool BF16OUT>
__global__ __launch_bounds__(256) void k_dequant_variant(const uint8_t* __restrict__ codes,
                                                         const uint8_t* __restrict__ scales,
                                                         const float* __restrict__ tensor_scale, int64_t n16,
                                                         void* __restrict__ y) {
  using D = Var<V>;
  constexpr int BITS = D::kBits;
  constexpr int STEPS = 4;   // 4 steps of 8 elements: 32 per lane, 2048 per wave
  __shared__ VarRestore rt;
  if (threadIdx.x < (1u << BITS))
    rt.r[threadIdx.x ^ (1u << (BITS - 1))] =   // indexed by the two's complement code
        (float)((int)threadIdx.x - (1 << (BITS - 1))) * (D::kDirect ? 1.0f : D::kCinv);
  __syncthreads();
  const int64_t n = n16 * 16;
  const int lane = threadIdx.x & 63;
  const int64_t e0 = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * (64 * 8 * STEPS) + lane * 8;
  const float gs = *tensor_scale, rgs = __fdiv_rn(1.0f, gs);
  // loads first (clamped addresses), so all of them are in flight together
  Codes16 c[STEPS];
  uint32_t sb[STEPS];
#pragma unroll
  for (int j = 0; j < STEPS; ++j) {
    const int64_t g = min(e0 + (int64_t)j * 512, n - 8) >> 4;
    c[j].w[0] = c[j].w[1] = c[j].w[2] = 0u;
    if constexpr (BITS == 3) {
      const uint16_t* src = reinterpret_cast<const uint16_t*>(codes + g * 6);
      c[j].w[0] = (uint32_t)src[0] | ((uint32_t)src[1] << 16);
      c[j].w[1] = src[2];
    } else {
      const uint32_t* src = reinterpret_cast<const uint32_t*>(codes + g * 12);
      c[j].w[0] = src[0];
      c[j].w[1] = src[1];
      c[j].w[2] = src[2];
    }
    sb[j] = scales[g];
  }
#pragma unroll
  for (int j = 0; j < STEPS; ++j) {
    const int64_t e = e0 + (int64_t)j * 512;
    if (e >= n) break;
    const int half = (int)((e >> 3) & 1);
    const float s = e4m3_decode(sb[j] & 0x7Fu);
    const bool is_int = !D::kFp || (sb[j] & 0x80u);
    float rv[8], out[8];
    f32x32v d6;
    if constexpr (BITS == 6) {
      u32x6v cw;
      cw[0] = cw[3] = c[j].w[0];
      cw[1] = cw[4] = c[j].w[1];
      cw[2] = cw[5] = c[j].w[2];
      d6 = fp6_decode32<0>(cw);   // FP6 E2M3 values of the block's codes (16..31 repeat them)
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const uint32_t code0 = get16<BITS>(c[j], k), code1 = get16<BITS>(c[j], 8 + k);
      const uint32_t code = half ? code1 : code0;
      if (is_int) {
        rv[k] = rt.r[code];
      } else if constexpr (BITS == 3) {
        const uint32_t mc = code & 3u;
        const float mag = mc ? __uint_as_float((mc + 126u) << 23) : 0.0f;
        rv[k] = (code & 4u) ? -mag : mag;
      } else {
        rv[k] = half ? d6[8 + k] : d6[k];
      }
    }
    const float ratio = s * rgs;
    if (ratio >= 0x1p-98f && ratio <= 0x1p+96f) {
#pragma unroll
      for (int k = 0; k < 8; ++k) out[k] = div_rs(rv[k] * s, gs, rgs);
    } else {
#pragma unroll
      for (int k = 0; k < 8; ++k) out[k] = __fdiv_rn(rv[k] * s, gs);
    }
    if constexpr (BF16OUT) {
      typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
      uint32_t o[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        o[i] = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{out[2 * i], out[2 * i + 1]}, bf16x2v));
      // a wave's store covers 1 KiB of whole lines, written once: non-temporal
      __builtin_nontemporal_store(u32x4_t{o[0], o[1], o[2], o[3]}, reinterpret_cast<u32x4_t*>(static_cast<uint16_t*>(y) + e));
    } else {
      float4* d = reinterpret_cast<float4*>(static_cast<float*>(y) + e);
      d[0] = make_float4(out[0], out[1], out[2], out[3]);
      d[1] = make_float4(out[4], out[5], out[6], out[7]);
    }
  }
}

template <int V>
static void launch_variant_v(const void* x, int dtype, int64_t n16, const AmaxSource& amax, float* ts,
                             uint8_t* codes, uint8_t* scales, hipStream_t st) {
  const int grid = (int)((n16 + 256 * kVarBlocks - 1) / (256 * kVarBlocks));
  if (dtype == 1)
    k_variant<uint16_t, V><<<grid, 256, 0, st>>>(static_cast<const uint16_t*>(x), n16, amax, ts, codes, scales);
  else
    k_variant<float, V><<<grid, 256, 0, st>>>(static_cast<const float*>(x), n16, amax, ts, codes, scales);
}

void launch_variant(int var, const void* x, int dtype, int64_t rows, int64_t cols, const AmaxSource& amax,
                    float* tensor_scale, uint8_t* codes, uint8_t* scales, hipStream_t st) {
  const int64_t n16 = rows * cols / 16;
  switch (var) {
    case 0: launch_variant_v<0>(x, dtype, n16, amax, tensor_scale, codes, scales, st); break;
    case 1: launch_variant_v<1>(x, dtype, n16, amax, tensor_scale, codes, scales, st); break;
    case 2: launch_variant_v<2>(x, dtype, n16, amax, tensor_scale, codes, scales, st); break;
    case 3: launch_variant_v<3>(x, dtype, n16, amax, tensor_scale, codes, scales, st); break;
    default: launch_variant_v<4>(x, dtype, n16, amax, tensor_scale, codes, scales, st); break;
  }
}

template <int V>
static void launch_dequant_variant_v(const uint8_t* codes, const uint8_t* scales, const float* ts, int64_t n16,
                                     int out_dtype, void* y, hipStream_t st) {
  const int grid = (int)((n16 * 16 + 8191) / 8192);   // 2048 elements per wave, 4 waves
  if (out_dtype == 1) k_dequant_variant<V, true><<<grid, 256, 0, st>>>(codes, scales, ts, n16, y);
  else k_dequant_variant<V, false><<<grid, 256, 0, st>>>(codes, scales, ts, n16, y);
}

void launch_dequant_variant(int var, const uint8_t* codes, const uint8_t* scales, const float* tensor_scale,
                            int64_t rows, int64_t cols, int out_dtype, void* y, hipStream_t st) {
  const int64_t n16 = rows * cols / 16;
  switch (var) {
    // the 4-bit formats decode as NVFP4 (Four Over Six: E2M1 on E4M3 scales) and as IF4's
    // INT4 blocks without the 6/7 factor (NVINT4), in k_dequant's store-coalesced layout
    case 0: launch_dequant(0, codes, scales, tensor_scale, rows, cols, out_dtype, y, st); break;
    case 1: launch_dequant(4, codes, scales, tensor_scale, rows, cols, out_dtype, y, st); break;
    case 2: launch_dequant_variant_v<2>(codes, scales, tensor_scale, n16, out_dtype, y, st); break;
    case 3: launch_dequant(3, codes, scales, tensor_scale, rows, cols, out_dtype, y, st); break;   // IF4
    default: launch_dequant_variant_v<4>(codes, scales, tensor_scale, n16, out_dtype, y, st); break;
  }
}

}  // namespace fp4q
