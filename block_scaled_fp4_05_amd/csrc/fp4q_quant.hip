// fp4q_quant.hip -- quantize / dequantize kernels of libfp4q (no RHT).
//
// Operations (pages cited by address and section):
//  * NVFP4 1x16, row-wise and the transposed column-wise layout:
//    qiita.com/nishiha/items/b98c2b931d588c4c81d5, "Blockwise", "誤差逆伝播と転置",
//    "scaleの導出"; stochastic rounding: same page, "確率的丸め".
//  * NVFP4 16x16 (weights): same page, "2D scaling".
//  * MXFP4 32 + E8M0: ultralytics.com/ja/glossary/fp4, "FP4の仕組み"; RNE of the
//    E8M0 conversion: blog.ast.moe/blog/2026-09-24, "FP6で隣り合う値の間隔を見てみる".
//  * IF4: gist.science/ja/paper/2603.28765, "2. 提案手法：IF4".
//
// Every kernel is memory-streaming: 16-byte loads, per-block reductions in
// registers or across neighbouring lanes (DPP), and packed nibble stores.
#include "fp4q_dev.hpp"
#include "fp4q_internal.hpp"

namespace fp4q {

// ===========================================================================
// Tensor amax
// ===========================================================================

__global__ void k_zero1(float* p) { *p = 0.0f; }

// Same-address device atomics serialize at the memory side, so each workgroup
// reduces its share (DPP/shuffle within waves, LDS across waves) and issues a single
// atomic; the grid is sized to about one 1024-thread workgroup per CU.
template <typename T>
__global__ __launch_bounds__(1024) void k_amax(const T* __restrict__ x, int64_t n8, AmaxSink sink) {
  __shared__ float wmax[16];
  float m = 0.0f;
  const int64_t stride = (int64_t)gridDim.x * 1024;
  int64_t g = (int64_t)blockIdx.x * 1024 + threadIdx.x;
  for (; g + 3 * stride < n8; g += 4 * stride) {
    float a[8], b[8], c[8], d[8];
    load8(x, g * 8, a);
    load8(x, (g + stride) * 8, b);
    load8(x, (g + 2 * stride) * 8, c);
    load8(x, (g + 3 * stride) * 8, d);
#pragma unroll
    for (int k = 0; k < 8; ++k)
      m = __builtin_fmaxf(m, __builtin_fmaxf(__builtin_fmaxf(__builtin_fabsf(a[k]), __builtin_fabsf(b[k])),
                                             __builtin_fmaxf(__builtin_fabsf(c[k]), __builtin_fabsf(d[k]))));
  }
  for (; g < n8; g += stride) {
    float a[8];
    load8(x, g * 8, a);
#pragma unroll
    for (int k = 0; k < 8; ++k) m = __builtin_fmaxf(m, __builtin_fabsf(a[k]));
  }
  m = wave_max(m);
  if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    float bm = 0.0f;
    const int nw = (int)(blockDim.x >> 6);
    for (int w = 0; w < nw; ++w) bm = __builtin_fmaxf(bm, wmax[w]);
    post_amax(sink, bm);
  }
}

// amax over a tail of fewer than 8 elements (only for fp4q_amax on odd sizes)
template <typename T>
__global__ void k_amax_tail(const T* __restrict__ x, int64_t start, int64_t n, AmaxSink sink) {
  int64_t i = start + threadIdx.x;
  float m = 0.0f;
  if (i < n) {
    if constexpr (sizeof(T) == 2) m = __builtin_fabsf(__uint_as_float((uint32_t)x[i] << 16));
    else m = __builtin_fabsf(x[i]);
  }
  m = wave_max(m);
  if (threadIdx.x == 0) post_amax(sink, m);
}

// Large tensors: two 256-thread workgroups per CU, each thread keeping four
// non-temporal 16-byte loads in flight, and the maximum taken on magnitude bits
// (|x| orders like its bits with the sign cleared; bf16 two at a time).
template <typename T>
__global__ __launch_bounds__(256) void k_amax_wide(const u32x4_t* __restrict__ x, int64_t n16, AmaxSink sink) {
  __shared__ float wm[4];
  typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
  const int64_t stride = (int64_t)gridDim.x * 256;
  int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x;
  uint32_t m32 = 0;
  u16x2 m16 = {0, 0};
  auto fold = [&](const u32x4_t v) {
    if constexpr (sizeof(T) == 2) {
      m16 = __builtin_elementwise_max(m16, __builtin_bit_cast(u16x2, v.x & 0x7FFF7FFFu));
      m16 = __builtin_elementwise_max(m16, __builtin_bit_cast(u16x2, v.y & 0x7FFF7FFFu));
      m16 = __builtin_elementwise_max(m16, __builtin_bit_cast(u16x2, v.z & 0x7FFF7FFFu));
      m16 = __builtin_elementwise_max(m16, __builtin_bit_cast(u16x2, v.w & 0x7FFF7FFFu));
    } else {
      m32 = max(m32, max(max(v.x & 0x7FFFFFFFu, v.y & 0x7FFFFFFFu), max(v.z & 0x7FFFFFFFu, v.w & 0x7FFFFFFFu)));
    }
  };
  for (; g + 3 * stride < n16; g += 4 * stride) {
    u32x4_t v[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) v[k] = __builtin_nontemporal_load(x + g + k * stride);
#pragma unroll
    for (int k = 0; k < 4; ++k) fold(v[k]);
  }
  for (; g < n16; g += stride) fold(__builtin_nontemporal_load(x + g));
  float f;
  if constexpr (sizeof(T) == 2) f = __uint_as_float((uint32_t)max(m16.x, m16.y) << 16);
  else f = __uint_as_float(m32);
  f = wave_max(f);
  if ((threadIdx.x & 63) == 0) wm[threadIdx.x >> 6] = f;
  __syncthreads();
  if (threadIdx.x == 0) post_amax(sink, __builtin_fmaxf(__builtin_fmaxf(wm[0], wm[1]), __builtin_fmaxf(wm[2], wm[3])));
}

static int amax_grid(int64_t n8) {
  int64_t blocks = (n8 + 1023) / 1024;
  return (int)(blocks < 256 ? (blocks > 0 ? blocks : 1) : 256);
}

static int num_cus();

template <typename T>
static void launch_amax_t(const void* x, int64_t n, const AmaxSink& sink, hipStream_t st) {
  const T* xp = static_cast<const T*>(x);
  if (!sink.tp) k_zero1<<<1, 1, 0, st>>>(sink.f);
  if ((int64_t)sizeof(T) * n >= ((int64_t)128 << 20)) {
    const int64_t per16 = 16 / sizeof(T), n16 = n / per16;
    k_amax_wide<T><<<2 * num_cus(), 256, 0, st>>>(static_cast<const u32x4_t*>(x), n16, sink);
    if (n16 * per16 < n) k_amax_tail<T><<<1, 64, 0, st>>>(xp, n16 * per16, n, sink);
    return;
  }
  int64_t n8 = n / 8;
  if (n8 > 0) k_amax<T><<<amax_grid(n8), 1024, 0, st>>>(xp, n8, sink);
  if (n8 * 8 < n) k_amax_tail<T><<<1, 64, 0, st>>>(xp, n8 * 8, n, sink);
}

void launch_amax_to(const void* x, int dtype, int64_t n, const AmaxSink& sink, hipStream_t st) {
  if (dtype == 1) launch_amax_t<uint16_t>(x, n, sink, st);
  else launch_amax_t<float>(x, n, sink, st);
}

void launch_amax(const void* x, int dtype, int64_t n, float* amax, hipStream_t st) {
  launch_amax_to(x, dtype, n, AmaxSink{amax, nullptr}, st);
}

// ===========================================================================
// NVFP4 1x16, row-wise and/or column-wise, one pass over x.
//
// A workgroup of four waves owns a 128 x 128 tile; wave w takes rows 32w..32w+31.
// Lane layout inside a wave: quads of four lanes own a 16x16 sub-tile; lane bit 0
// picks the upper or lower 8 rows and lane bit 1 the left or right 8 columns, so
// every lane holds an 8x8 micro-tile as raw input words.  A row block (16 columns)
// is the lane pair (lane ^ 2) and a column block (16 rows) the pair (lane ^ 1): both
// block maxima are one DPP max away.  t = x*gs is formed once per element and
// serves both directions.
//
// Codes and scales are staged in LDS for the whole tile, so every column's 64 bytes
// of codes and 8 scale bytes leave contiguously, and rows' outputs leave as 16-byte
// stores.  Tiles are dealt in groups of 16 x 16 tiles (2048 x 2048 elements): each
// XCD (block b runs on XCD b % 8) gets a contiguous run of the group-major tile
// sequence, so output cache lines that several tiles share are completed inside one
// XCD's L2 while it works on the group.
// ===========================================================================

template <typename T> struct Raw8x8;
// Loads are unconditional, so no branch forces an early wait on them: rows past the
// end and columns past the end read the last valid row / column group instead.  Such
// values only ever enter row or column blocks whose outputs are not stored (blocks
// never straddle the matrix edge), so they cannot change a stored code.
// The input is read exactly once, so its loads are marked non-temporal: they do not
// displace the output lines that neighbouring tiles are still completing in L2.

template <> struct Raw8x8<uint16_t> {
  uint4 r[8];
  __device__ __forceinline__ void load(const uint16_t* __restrict__ x, int row0, int col0, int rows, int cols) {
    const int c = min(col0, cols - 8);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const u32x4_t v = __builtin_nontemporal_load(
          reinterpret_cast<const u32x4_t*>(x + (int64_t)min(row0 + i, rows - 1) * cols + c));
      r[i] = make_uint4(v.x, v.y, v.z, v.w);
    }
  }
  __device__ __forceinline__ uint32_t word(int i, int k) const {
    return k == 0 ? r[i].x : k == 1 ? r[i].y : k == 2 ? r[i].z : r[i].w;
  }
  // element (i, j) of the micro-tile times gs
  __device__ __forceinline__ float at(int i, int j, float gs) const {
    const uint32_t w = word(i, j >> 1);
    return ((j & 1) ? bf16_hi(w) : bf16_lo(w)) * gs;
  }
};
template <> struct Raw8x8<float> {
  float4 r[16];
  __device__ __forceinline__ void load(const float* __restrict__ x, int row0, int col0, int rows, int cols) {
    const int c = min(col0, cols - 8);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float* p = x + (int64_t)min(row0 + i, rows - 1) * cols + c;
      const f32x4_t a = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(p));
      const f32x4_t b = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(p + 4));
      r[2 * i] = make_float4(a.x, a.y, a.z, a.w);
      r[2 * i + 1] = make_float4(b.x, b.y, b.z, b.w);
    }
  }
  __device__ __forceinline__ float at(int i, int j, float gs) const {
    const float4 v = r[2 * i + (j >> 2)];
    const int k = j & 3;
    return (k == 0 ? v.x : k == 1 ? v.y : k == 2 ? v.z : v.w) * gs;
  }
};

// Maxima of |x| over the lane's 16-element blocks, found from the raw words before
// the tensor scale is known (the one-pass kernel does this while it waits for the
// other workgroups): for row i (i = 0..7) of the lane's micro-tile the row block
// (16 columns, this lane and lane ^ 2), for column j the column block (16 rows, this
// lane and lane ^ 1).  Then max|fl(x*gs)| over a block = fl(bamax*gs), since the
// product rounds monotonically.  bf16 keeps the magnitude bits two per word.
template <typename T> struct BlockMax;
template <> struct BlockMax<uint16_t> {
  uint32_t row[4], col[4];   // row[k]: rows 2k (low half), 2k+1; col[k]: columns 2k, 2k+1
  __device__ __forceinline__ void compute(const Raw8x8<uint16_t>& raw) {
    typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
    u16x2 m[8][4];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int k = 0; k < 4; ++k) m[i][k] = __builtin_bit_cast(u16x2, raw.word(i, k) & 0x7FFF7FFFu);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      uint32_t r[2];
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int i = 2 * k + e;
        const u16x2 a = __builtin_elementwise_max(__builtin_elementwise_max(m[i][0], m[i][1]),
                                                  __builtin_elementwise_max(m[i][2], m[i][3]));
        r[e] = a.x > a.y ? a.x : a.y;
      }
      const uint32_t w = r[0] | (r[1] << 16);
      const uint32_t o = (uint32_t)__builtin_amdgcn_mov_dpp((int)w, 0x4E, 0xF, 0xF, false);   // lane ^ 2
      row[k] = __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(u16x2, w),
                                                                       __builtin_bit_cast(u16x2, o)));
      u16x2 c = m[0][k];
#pragma unroll
      for (int i = 1; i < 8; ++i) c = __builtin_elementwise_max(c, m[i][k]);
      const uint32_t cw = __builtin_bit_cast(uint32_t, c);
      const uint32_t co = (uint32_t)__builtin_amdgcn_mov_dpp((int)cw, 0xB1, 0xF, 0xF, false);   // lane ^ 1
      col[k] = __builtin_bit_cast(uint32_t, __builtin_elementwise_max(c, __builtin_bit_cast(u16x2, co)));
    }
  }
  __device__ __forceinline__ float rowmax(int i) const {
    return __uint_as_float((i & 1) ? (row[i >> 1] & 0xFFFF0000u) : (row[i >> 1] << 16));
  }
  __device__ __forceinline__ float colmax(int j) const {
    return __uint_as_float((j & 1) ? (col[j >> 1] & 0xFFFF0000u) : (col[j >> 1] << 16));
  }
  // maximum over every element of the micro-tile (any block covers its rows)
  __device__ __forceinline__ float lanemax() const {
    uint32_t m = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) m = max(m, max(row[k] << 16, row[k] & 0xFFFF0000u));
    return __uint_as_float(m);
  }
};
template <> struct BlockMax<float> {
  uint32_t row[8], col[8];   // magnitude bits
  __device__ __forceinline__ void compute(const Raw8x8<float>& raw) {
    uint32_t m[8][8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < 8; ++j) m[i][j] = __float_as_uint(raw.at(i, j, 1.0f)) & 0x7FFFFFFFu;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      uint32_t a = 0;
#pragma unroll
      for (int j = 0; j < 8; ++j) a = max(a, m[i][j]);
      row[i] = max(a, (uint32_t)__builtin_amdgcn_mov_dpp((int)a, 0x4E, 0xF, 0xF, false));
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      uint32_t a = 0;
#pragma unroll
      for (int i = 0; i < 8; ++i) a = max(a, m[i][j]);
      col[j] = max(a, (uint32_t)__builtin_amdgcn_mov_dpp((int)a, 0xB1, 0xF, 0xF, false));
    }
  }
  __device__ __forceinline__ float rowmax(int i) const { return __uint_as_float(row[i]); }
  __device__ __forceinline__ float colmax(int j) const { return __uint_as_float(col[j]); }
  __device__ __forceinline__ float lanemax() const {
    uint32_t m = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) m = max(m, row[i]);
    return __uint_as_float(m);
  }
};

// Staging of one 128 x 128 tile's outputs.  A row's 64 bytes of codes sit at dword
// r*16 + (r/8)*16 and a column's at c*16 + (c/8)*4: the padding after every eight
// rows / columns sends the lanes of one 4-byte write (four row groups, or sixteen
// column groups, at one i or j) to distinct banks, and it depends on r/8 and c/8 only,
// which are fixed for a lane's eight rows and columns, so the row or column index
// is a constant offset from one per-lane base.  16-byte chunks stay aligned.
struct TileStage {
  uint32_t rc[128 * 16 + 16 * 16];   // row codes: 128 rows x 64 B, 64 B pad per 8 rows
  uint32_t cc[128 * 16 + 16 * 4];    // column codes: 128 columns x 64 B (4 chunks of 32 tokens), 16 B pad per 8
  uint8_t rs[1024];                  // row scales: 128 rows x 8 blocks
  uint8_t cs[1024];                  // column scales: 128 columns x 8 blocks
};

// row r (0..127), 4-byte piece p (0..15) of its 64 bytes -> dword index in rc
__device__ __forceinline__ int rc_dword(int r, int p) { return r * 16 + (r >> 3) * 16 + p; }
// column c (0..127), 16-byte piece w (0..3, tokens 32w..32w+31), 4-byte part p
__device__ __forceinline__ int cc_dword(int c, int w, int p) { return c * 16 + (c >> 3) * 4 + w * 4 + p; }

__device__ __forceinline__ void store_u8x8(uint8_t* dst, uint2 v, int nvalid, bool aligned8) {
  if (nvalid >= 8 && aligned8) {
    *reinterpret_cast<uint2*>(dst) = v;
  } else {
    for (int e = 0; e < 8 && e < nvalid; ++e) dst[e] = (uint8_t)((e < 4 ? v.x : v.y) >> (8 * (e & 3)));
  }
}

// This lane's 8x8 micro-tile of tile (trow0, tcol0).
template <typename T>
__device__ __forceinline__ void nvfp4_tile_load(const T* __restrict__ x, int trow0, int tcol0, int rows, int cols,
                                                Raw8x8<T>& raw) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int q = lane >> 2, h = (lane >> 1) & 1, vv = lane & 1;
  const int row0 = trow0 + wave * 32 + (q >> 3) * 16 + vv * 8, col0 = tcol0 + (q & 7) * 16 + h * 8;
  raw.load(x, row0, col0, rows, cols);
}

template <typename T, bool ROW, bool COL, bool SR, bool PRE = false>
__device__ __forceinline__ void nvfp4_tile(Raw8x8<T>& raw, int trow0, int tcol0, int rows, int cols, float gs,
                                           TileStage& st, const RecipTable& rtab, const BlockMax<T>* bm,
                                           uint8_t* __restrict__ rcodes, uint8_t* __restrict__ rscales,
                                           uint8_t* __restrict__ ccodes, uint8_t* __restrict__ cscales, uint32_t k0,
                                           uint32_t k1) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int q = lane >> 2, h = (lane >> 1) & 1, vv = lane & 1, qr = q >> 3, qc = q & 7;
  const int lrow0 = wave * 32 + qr * 16 + vv * 8, lcol0 = qc * 16 + h * 8;   // within the tile
  const int row0 = trow0 + lrow0, col0 = tcol0 + lcol0;

  // staging addresses of row lrow0 + i and column lcol0 + j: base + constant
  uint32_t* const rc_lane = &st.rc[rc_dword(lrow0, 2 * qc + h)];
  uint8_t* const rs_lane = &st.rs[lrow0 * 8 + qc];
  uint32_t* const cc_lane = &st.cc[cc_dword(lcol0, wave, 2 * qr + vv)];
  uint8_t* const cs_lane = &st.cs[lcol0 * 8 + 2 * wave + qr];

  // t = fl(x*gs) for the lane's 64 elements, formed once for both directions
  float t[8][8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) t[i][j] = raw.at(i, j, gs);

  if constexpr (ROW) {
    const uint64_t idx0 = (uint64_t)row0 * (uint64_t)cols + (uint64_t)col0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float m = 0.0f;
      if constexpr (PRE) {
        m = bm->rowmax(i) * gs;
      } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) m = __builtin_fmaxf(m, __builtin_fabsf(t[i][j]));
        m = lane_xor_max<2>(m);
      }
      const uint32_t code = nvfp4_scale_code(m);
      const RecipPair rp = rtab.r[code];
      float v[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] = div2(t[i][j], rp);
      uint32_t w;
      if constexpr (SR) {
        uint32_t rr[8];
        sr_draws8((idx0 + (uint64_t)i * (uint64_t)cols) >> 3, 0u, k0, k1, rr);
        w = pack8_sr(v, rr, 1.0f);
      } else {
        w = pack8_rtn(v, 1.0f);
      }
      rc_lane[i * 16] = w;
      rs_lane[i * 8] = (uint8_t)code;   // both lanes of the block write the same byte
    }
  }
  if constexpr (COL) {
    const uint64_t idx0 = (uint64_t)col0 * (uint64_t)rows + (uint64_t)row0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      float m = 0.0f;
      if constexpr (PRE) {
        m = bm->colmax(j) * gs;
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) m = __builtin_fmaxf(m, __builtin_fabsf(t[i][j]));
        m = lane_xor_max<1>(m);
      }
      const uint32_t code = nvfp4_scale_code(m);
      const RecipPair rp = rtab.r[code];
      float v[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = div2(t[i][j], rp);
      uint32_t w;
      if constexpr (SR) {
        uint32_t rr[8];
        sr_draws8((idx0 + (uint64_t)j * (uint64_t)rows) >> 3, 1u, k0, k1, rr);
        w = pack8_sr(v, rr, 1.0f);
      } else {
        w = pack8_rtn(v, 1.0f);
      }
      cc_lane[j * 16] = w;
      cs_lane[j * 8] = (uint8_t)code;   // both lanes of the block write the same byte
    }
  }
  lds_barrier();
  const int tid = threadIdx.x;
  // Interior tile of a 128-aligned matrix (uniform test): every store is whole and
  // aligned, so none needs a per-lane bounds check.
  if (((rows | cols) & 127) == 0 && trow0 + 128 <= rows && tcol0 + 128 <= cols) {
    if constexpr (ROW) {
      const int half_cols = cols >> 1, nb = cols >> 4;
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const int ch = tid + 256 * k, r = ch >> 2, c4 = ch & 3;
        *reinterpret_cast<uint4*>(rcodes + (int64_t)(trow0 + r) * half_cols + ((tcol0 + c4 * 32) >> 1)) =
            *reinterpret_cast<const uint4*>(&st.rc[rc_dword(r, c4 * 4)]);
      }
      if (tid < 128)
        *reinterpret_cast<uint2*>(rscales + (int64_t)(trow0 + tid) * nb + (tcol0 >> 4)) =
            *reinterpret_cast<const uint2*>(&st.rs[tid * 8]);
    }
    if constexpr (COL) {
      const int half_rows = rows >> 1, nb = rows >> 4;
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const int ch = tid + 256 * k, c = ch >> 2, w = ch & 3;
        *reinterpret_cast<uint4*>(ccodes + (int64_t)(tcol0 + c) * half_rows + ((trow0 + 32 * w) >> 1)) =
            *reinterpret_cast<const uint4*>(&st.cc[cc_dword(c, w, 0)]);
      }
      if (tid < 128)
        *reinterpret_cast<uint2*>(cscales + (int64_t)(tcol0 + tid) * nb + (trow0 >> 4)) =
            *reinterpret_cast<const uint2*>(&st.cs[tid * 8]);
    }
    return;
  }
  if constexpr (ROW) {
    const int half_cols = cols >> 1, nb = cols >> 4;
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int ch = tid + 256 * k;                        // chunk: row ch / 4, 32 columns
      const int r = ch >> 2, c4 = ch & 3;
      const uint4 w = *reinterpret_cast<const uint4*>(&st.rc[rc_dword(r, c4 * 4)]);
      const int grow = trow0 + r, gcol = tcol0 + c4 * 32;   // first column of this 32-column chunk
      if (grow < rows && gcol < cols) {
        uint8_t* dst = rcodes + (int64_t)grow * half_cols + (gcol >> 1);   // 8-byte aligned
        if (gcol + 32 > cols) {
          *reinterpret_cast<uint2*>(dst) = make_uint2(w.x, w.y);           // 16 valid columns
        } else if ((half_cols & 15) == 0) {
          *reinterpret_cast<uint4*>(dst) = w;
        } else {
          reinterpret_cast<uint2*>(dst)[0] = make_uint2(w.x, w.y);
          reinterpret_cast<uint2*>(dst)[1] = make_uint2(w.z, w.w);
        }
      }
    }
    if (tid < 128) {
      const int grow = trow0 + tid, blk0 = tcol0 >> 4;
      if (grow < rows && blk0 < nb)
        store_u8x8(rscales + (int64_t)grow * nb + blk0, *reinterpret_cast<const uint2*>(&st.rs[tid * 8]),
                   nb - blk0, (nb & 7) == 0);
    }
  }
  if constexpr (COL) {
    const int half_rows = rows >> 1, nb = rows >> 4;
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int ch = tid + 256 * k;
      const int c = ch >> 2, w = ch & 3;
      const uint4 v = *reinterpret_cast<const uint4*>(&st.cc[cc_dword(c, w, 0)]);
      const int gcol = tcol0 + c, grow = trow0 + 32 * w;
      if (gcol < cols && grow + 16 <= rows) {
        uint8_t* dst = ccodes + (int64_t)gcol * half_rows + (grow >> 1);   // 8-byte aligned
        if (grow + 32 > rows) {
          *reinterpret_cast<uint2*>(dst) = make_uint2(v.x, v.y);
        } else if ((half_rows & 15) == 0) {
          *reinterpret_cast<uint4*>(dst) = v;
        } else {
          reinterpret_cast<uint2*>(dst)[0] = make_uint2(v.x, v.y);
          reinterpret_cast<uint2*>(dst)[1] = make_uint2(v.z, v.w);
        }
      }
    }
    if (tid < 128) {
      const int gcol = tcol0 + tid, blk0 = trow0 >> 4;
      if (gcol < cols && blk0 < nb)
        store_u8x8(cscales + (int64_t)gcol * nb + blk0, *reinterpret_cast<const uint2*>(&st.cs[tid * 8]),
                   nb - blk0, (nb & 7) == 0);
    }
  }
  // No second barrier: the caller alternates between two staging buffers, and the
  // next tile's barrier orders these reads before the buffer is written again.
}

// Tile t of the group-major sequence -> (tile row, tile column).
__device__ __forceinline__ void group_major_tile(int t, int tiles_r, int tiles_c, int& tr, int& tc) {
  constexpr int G = 16;
  const int full_rows_tiles = G * tiles_c;                 // tiles in one full group-row
  const int gr = t / full_rows_tiles;
  int rem = t - gr * full_rows_tiles;
  const int gh = min(G, tiles_r - gr * G);                 // height of this group-row
  const int gc = rem / (gh * G);
  const int gw = min(G, tiles_c - gc * G);
  rem -= gc * gh * G;
  tr = gr * G + rem / gw;
  tc = gc * G + rem % gw;
}

template <typename T, bool ROW, bool COL, bool SR>
__global__ __launch_bounds__(256) void k_nvfp4_tile(
    const T* __restrict__ x, int rows, int cols, int tiles_r, int tiles_c,
    AmaxSource amax, float* __restrict__ tensor_scale,
    uint8_t* __restrict__ rcodes, uint8_t* __restrict__ rscales,
    uint8_t* __restrict__ ccodes, uint8_t* __restrict__ cscales,
    uint32_t k0, uint32_t k1) {
  __shared__ TileStage stage[2];   // tile parity alternates the staging buffer
  __shared__ RecipTable rtab;
  fill_recip_table(rtab);
  __syncthreads();
  const float gs = tensor_scale_publish(amax, tensor_scale);

  // tiles of XCD x (blocks b with b % 8 == x) form the contiguous band
  // [x*per, (x+1)*per) of the group-major sequence; the band's blocks stride through it.
  const int total = tiles_r * tiles_c;
  const int nblk = gridDim.x, b = blockIdx.x;
  const int xcd = b & 7, nx = (nblk + 7 - xcd) >> 3, lb = b >> 3;
  const int per = (total + 7) >> 3;
  const int band0 = xcd * per, band1 = min(total, band0 + per);
  // ping-pong: the next tile's raw input is in flight while this one is computed
  int t = band0 + lb;
  if (t >= band1) return;
  Raw8x8<T> ra, rb;
  int tra, tca, trb, tcb;
  group_major_tile(t, tiles_r, tiles_c, tra, tca);
  nvfp4_tile_load<T>(x, tra * 128, tca * 128, rows, cols, ra);
  // Each step is written out twice (with and without the next load) so that the
  // compiler's wait before the compute only covers the current tile's loads.
  while (true) {
    const int t1 = t + nx;
    if (t1 < band1) {
      group_major_tile(t1, tiles_r, tiles_c, trb, tcb);
      nvfp4_tile_load<T>(x, trb * 128, tcb * 128, rows, cols, rb);
      nvfp4_tile<T, ROW, COL, SR>(ra, tra * 128, tca * 128, rows, cols, gs, stage[0], rtab, nullptr, rcodes, rscales, ccodes,
                                  cscales, k0, k1);
    } else {
      nvfp4_tile<T, ROW, COL, SR>(ra, tra * 128, tca * 128, rows, cols, gs, stage[0], rtab, nullptr, rcodes, rscales, ccodes,
                                  cscales, k0, k1);
      break;
    }
    const int t2 = t1 + nx;
    if (t2 < band1) {
      group_major_tile(t2, tiles_r, tiles_c, tra, tca);
      nvfp4_tile_load<T>(x, tra * 128, tca * 128, rows, cols, ra);
      nvfp4_tile<T, ROW, COL, SR>(rb, trb * 128, tcb * 128, rows, cols, gs, stage[1], rtab, nullptr, rcodes, rscales, ccodes,
                                  cscales, k0, k1);
    } else {
      nvfp4_tile<T, ROW, COL, SR>(rb, trb * 128, tcb * 128, rows, cols, gs, stage[1], rtab, nullptr, rcodes, rscales, ccodes,
                                  cscales, k0, k1);
      break;
    }
    t = t2;
  }
}

static int g_num_cus = 0;

static int num_cus() {
  if (g_num_cus == 0) {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0)
      g_num_cus = n;
    else
      g_num_cus = 256;
  }
  return g_num_cus;
}

template <typename T, bool ROW, bool COL, bool SR>
static void launch_nvfp4_t(const void* x, int64_t rows, int64_t cols, const AmaxSource& amax,
                           float* tensor_scale, uint8_t* rc, uint8_t* rs, uint8_t* cc, uint8_t* cs,
                           uint32_t k0, uint32_t k1, hipStream_t st) {
  const int tiles_r = (int)((rows + 127) / 128), tiles_c = (int)((cols + 127) / 128);
  const int total = tiles_r * tiles_c;
  const int want = num_cus() * 2;          // two resident 4-wave workgroups per CU, each walking tiles
  const int grid = total < want ? total : want;
  k_nvfp4_tile<T, ROW, COL, SR><<<grid, 256, 0, st>>>(static_cast<const T*>(x), (int)rows, (int)cols, tiles_r,
                                                      tiles_c, amax, tensor_scale, rc, rs, cc, cs, k0, k1);
}

template <typename T>
static void launch_nvfp4_dt(const void* x, int64_t rows, int64_t cols, unsigned layouts, bool sr,
                            const AmaxSource& amax, float* ts, uint8_t* rc, uint8_t* rs, uint8_t* cc,
                            uint8_t* cs, uint32_t k0, uint32_t k1, hipStream_t st) {
  const bool row = layouts & 1u, col = layouts & 2u;
#define FP4Q_NV(R, C, S) launch_nvfp4_t<T, R, C, S>(x, rows, cols, amax, ts, rc, rs, cc, cs, k0, k1, st)
  if (row && col) { if (sr) FP4Q_NV(true, true, true); else FP4Q_NV(true, true, false); }
  else if (row)   { if (sr) FP4Q_NV(true, false, true); else FP4Q_NV(true, false, false); }
  else            { if (sr) FP4Q_NV(false, true, true); else FP4Q_NV(false, true, false); }
#undef FP4Q_NV
}

void launch_nvfp4(const void* x, int dtype, int64_t rows, int64_t cols, unsigned layouts, bool sr,
                  const AmaxSource& amax, float* tensor_scale, uint8_t* rc, uint8_t* rs, uint8_t* cc,
                  uint8_t* cs, uint64_t seed, hipStream_t st) {
  const uint32_t k0 = (uint32_t)seed, k1 = (uint32_t)(seed >> 32);
  if (dtype == 1)
    launch_nvfp4_dt<uint16_t>(x, rows, cols, layouts, sr, amax, tensor_scale, rc, rs, cc, cs, k0, k1, st);
  else
    launch_nvfp4_dt<float>(x, rows, cols, layouts, sr, amax, tensor_scale, rc, rs, cc, cs, k0, k1, st);
}

// ===========================================================================
// NVFP4 1x16 with the tensor amax found in the same pass over x.
//
// The tensor scale depends on the maximum over the whole tensor, so a plain
// implementation reads x twice (amax, then quantize).  When the tensor fits in the
// register files of one co-resident grid (up to TPW tiles per workgroup), each
// workgroup instead loads all of its tiles once and keeps them in registers,
// publishes its partial maximum and meets the others at a grid-wide barrier; then
// every workgroup reduces the partial maxima itself, forms gs and quantizes its
// tiles from registers.  x leaves HBM once.
//
// The grid is sized from the occupancy query so that all workgroups are resident at
// once; then the exchange of partial maxima costs about a microsecond.  Correctness
// does not depend on it: every wait is bounded, and a workgroup whose wait runs out
// reads the missing part of x itself (see grid_max).
// ===========================================================================

// The one-pass kernel's exchange lives in a FusedArea of the caller's workspace.
// Values that cross workgroups travel in 64-bit slots holding (epoch << 32) | float
// bits: a reader that sees the current launch's epoch in a slot has the value in the
// same word, so no fence is needed and nothing is reset between launches.  The host
// numbers the launches on a workspace (epoch 1, 2, ...), so slots left by earlier
// launches never match.
//
// Workgroups form 8 groups, g = b % 8, and workgroup g leads group g: members post
// their slots, the leader combines them and posts the group maximum, and every
// workgroup reads the eight group maxima.  All of it is device-scope traffic, so no
// step relies on where a workgroup runs.

__device__ __forceinline__ float raw_absmax(const Raw8x8<uint16_t>& raw) {
  // |bf16| orders like its 15 magnitude bits, so a packed 16-bit max does two at once
  typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
  u16x2 m = {0, 0};
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int k = 0; k < 4; ++k)
      m = __builtin_elementwise_max(m, __builtin_bit_cast(u16x2, raw.word(i, k) & 0x7FFF7FFFu));
  const uint32_t b = m.x > m.y ? m.x : m.y;
  return __uint_as_float(b << 16);
}

__device__ __forceinline__ float raw_absmax(const Raw8x8<float>& raw) {
  float m = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i)
    m = __builtin_fmaxf(m, __builtin_fmaxf(__builtin_fmaxf(__builtin_fabsf(raw.r[i].x), __builtin_fabsf(raw.r[i].y)),
                                           __builtin_fmaxf(__builtin_fabsf(raw.r[i].z), __builtin_fabsf(raw.r[i].w))));
  return m;
}

// Maximum over the workgroup of a per-thread value (every thread gets the result).
__device__ __forceinline__ float block_max256(float v, float* red) {
  v = wave_max(v);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  v = __builtin_fmaxf(__builtin_fmaxf(red[0], red[1]), __builtin_fmaxf(red[2], red[3]));
  __syncthreads();
  return v;
}

__device__ __forceinline__ uint64_t pack_epoch(uint32_t epoch, float v) {
  return ((uint64_t)epoch << 32) | __float_as_uint(v);
}

// Device-scope (single-location coherent) load of a slot.
__device__ __forceinline__ uint64_t load_dev(const uint64_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Polls `slot` until it carries `epoch`, for at most `wait_iters` rounds of a short
// sleep (each at least 256 clocks).  Returns whether the value arrived (in *v).
__device__ __forceinline__ bool poll_slot(const uint64_t* slot, uint32_t epoch, uint32_t wait_iters, float* v) {
  uint64_t w = load_dev(slot);
  for (uint32_t it = 0; (uint32_t)(w >> 32) != epoch; ++it) {
    if (it >= wait_iters) return false;
    __builtin_amdgcn_s_sleep(4);
    w = load_dev(slot);
  }
  *v = __uint_as_float((uint32_t)w);
  return true;
}

// max|x| over the tiles start, start + stride, ... (< end) of the group-major sequence,
// by the whole workgroup; every thread gets the result.  Only the fallback uses it.
template <typename T>
__device__ __noinline__ float tiles_absmax(const T* __restrict__ x, int rows, int cols, int tiles_r, int tiles_c,
                                           int start, int stride, int end, float* red) {
  float m = 0.0f;
  for (int t = start; t < end; t += stride) {
    int tr, tc;
    group_major_tile(t, tiles_r, tiles_c, tr, tc);
    Raw8x8<T> r;
    nvfp4_tile_load<T>(x, tr * 128, tc * 128, rows, cols, r);
    m = __builtin_fmaxf(m, raw_absmax(r));
  }
  return block_max256(m, red);
}

struct GridMaxShared {
  float red[4];
  alignas(16) uint32_t miss[8];   // bit j: slot j of the current wait did not arrive in time
  float val;
};

// The eight miss words, read with two 16-byte LDS loads (one round trip).
__device__ __forceinline__ void read_miss(const GridMaxShared& sh, uint32_t (&w)[8]) {
  const uint4 lo = *reinterpret_cast<const uint4*>(&sh.miss[0]);
  const uint4 hi = *reinterpret_cast<const uint4*>(&sh.miss[4]);
  w[0] = lo.x; w[1] = lo.y; w[2] = lo.z; w[3] = lo.w;
  w[4] = hi.x; w[5] = hi.y; w[6] = hi.z; w[7] = hi.w;
}

// Grid-wide maximum of the workgroups' values v (thread 0's copy), returned to every
// thread.  Members post their slot in the group area; leader g collects the group's
// slots and posts the group maximum; every workgroup then reads the eight group
// maxima itself (eight lines, polled by eight lanes).
//
// No wait depends on other workgroups making progress for correctness: a slot that
// has not arrived after `wait_iters` polls is computed from x by the waiting
// workgroup itself (one workgroup's tiles, or a group's band).  With the whole grid
// resident, which the launch size is chosen for, no fallback runs; without it, the
// grid still finishes with the exact maximum.
template <typename T>
__device__ __forceinline__ float all_groups_max(FusedArea* ws, uint32_t epoch, uint32_t wait_iters,
                                                const T* __restrict__ x, int rows, int cols, int tiles_r,
                                                int tiles_c, GridMaxShared& sh) {
  const int tid = threadIdx.x;
  const int total = tiles_r * tiles_c, per = (total + 7) >> 3;
  if (tid < 8) sh.miss[tid] = 0u;
  __syncthreads();
  float t = 0.0f;
  if (tid < 8) {
    float u;
    if (poll_slot(&ws->group[tid][0], epoch, wait_iters, &u)) t = u;
    else atomicOr(&sh.miss[0], 1u << tid);
  }
  __syncthreads();
  const uint32_t miss = sh.miss[0];                  // uniform; one LDS read, not one per group
  for (int k = 0; k < 8; ++k)
    if (miss & (1u << k)) {
      t = __builtin_fmaxf(t, tiles_absmax<T>(x, rows, cols, tiles_r, tiles_c, k * per, 1, min(total, (k + 1) * per),
                                             sh.red));
      if (tid == 0) __hip_atomic_fetch_add(&ws->fallbacks[0], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  return block_max256(t, sh.red);
}

template <typename T>
__device__ __forceinline__ float grid_max(FusedArea* ws, float v, uint32_t epoch, uint32_t wait_iters,
                                          const T* __restrict__ x, int rows, int cols, int tiles_r, int tiles_c,
                                          GridMaxShared& sh) {
  const int b = blockIdx.x, nwg = gridDim.x, g = b & 7, ng = nwg >> 3;
  const int tid = threadIdx.x;
  const int total = tiles_r * tiles_c, per = (total + 7) >> 3;
  uint64_t* local = ws->local[g];
  if (tid < 8) sh.miss[tid] = 0u;
  if (tid == 0 && b >= 8)
    __hip_atomic_store(&local[b >> 3], pack_epoch(epoch, v), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  if (b < 8) {                                        // leader of group g == b
    float m = v;
    for (int j = 1 + tid; j < ng; j += 256) {
      float u;
      if (poll_slot(&local[j], epoch, wait_iters, &u)) m = __builtin_fmaxf(m, u);
      else atomicOr(&sh.miss[j >> 5], 1u << (j & 31));
    }
    __syncthreads();
    // miss[] is shared, so the words are uniform; read them at once, since a loop that
    // re-read LDS per member would cost one LDS round trip per member
    uint32_t mw[8];
    read_miss(sh, mw);
    if ((mw[0] | mw[1] | mw[2] | mw[3] | mw[4] | mw[5] | mw[6] | mw[7]) != 0u) {
      for (int w = 0; w < 8; ++w)
        for (uint32_t bits = mw[w]; bits != 0u; bits &= bits - 1u) {
          const int j = w * 32 + __builtin_ctz(bits);
          const int band0 = g * per;
          m = __builtin_fmaxf(m, tiles_absmax<T>(x, rows, cols, tiles_r, tiles_c, band0 + j, ng,
                                                 min(total, band0 + per), sh.red));
          if (tid == 0) __hip_atomic_fetch_add(&ws->fallbacks[0], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
    m = block_max256(m, sh.red);
    if (tid == 0)
      __hip_atomic_store(&ws->group[g][0], pack_epoch(epoch, m), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  return all_groups_max<T>(ws, epoch, wait_iters, x, rows, cols, tiles_r, tiles_c, sh);
}

// Tile K, then K+1, ... with compile-time indices, so the raw tiles stay in registers.
template <typename T> constexpr int kBlockMaxWords = sizeof(BlockMax<T>) / 4;

template <typename T, int TPW, bool ROW, bool COL, bool SR, int K>
__device__ __forceinline__ void fused_phase2(Raw8x8<T> (&raw)[TPW],
                                             const uint32_t (&bmw)[TPW][kBlockMaxWords<T>][256],
                                             const int (&tr)[TPW], const int (&tc)[TPW],
                                             const bool (&ok)[TPW], int rows, int cols, float gs, TileStage (&stage)[2],
                                             const RecipTable& rtab, uint8_t* __restrict__ rcodes,
                                             uint8_t* __restrict__ rscales, uint8_t* __restrict__ ccodes,
                                             uint8_t* __restrict__ cscales, uint32_t k0, uint32_t k1) {
  if (ok[K]) {
    BlockMax<T> bm;
    uint32_t* w = reinterpret_cast<uint32_t*>(&bm);
#pragma unroll
    for (int e = 0; e < kBlockMaxWords<T>; ++e) w[e] = bmw[K][e][threadIdx.x];
    nvfp4_tile<T, ROW, COL, SR, true>(raw[K], tr[K] * 128, tc[K] * 128, rows, cols, gs, stage[K & 1], rtab, &bm,
                                      rcodes, rscales,
                                ccodes, cscales, k0, k1);
  }
  if constexpr (K + 1 < TPW)
    fused_phase2<T, TPW, ROW, COL, SR, K + 1>(raw, bmw, tr, tc, ok, rows, cols, gs, stage, rtab, rcodes, rscales, ccodes,
                                              cscales, k0, k1);
}

template <typename T, int TPW, bool ROW, bool COL, bool SR>
__global__ __launch_bounds__(256) void k_nvfp4_fused(
    const T* __restrict__ x, int rows, int cols, int tiles_r, int tiles_c, FusedArea* __restrict__ ws,
    uint32_t epoch, uint32_t wait_iters,
    float* __restrict__ amax_out, float* __restrict__ tensor_scale,
    uint8_t* __restrict__ rcodes, uint8_t* __restrict__ rscales,
    uint8_t* __restrict__ ccodes, uint8_t* __restrict__ cscales, uint32_t k0, uint32_t k1) {
  __shared__ TileStage stage[2];   // tile parity alternates the staging buffer
  __shared__ RecipTable rtab;
  __shared__ GridMaxShared gsh;
  fill_recip_table(rtab);

  // Same band layout as the streaming kernel: XCD x owns a contiguous run of the
  // group-major tile sequence and its nx workgroups take every nx-th tile of it.
  const int total = tiles_r * tiles_c;
  const int nwg = gridDim.x, b = blockIdx.x;
  const int xcd = b & 7, nx = (nwg + 7 - xcd) >> 3, lb = b >> 3;
  const int per = (total + 7) >> 3;
  const int band0 = xcd * per, band1 = min(total, band0 + per);
  const int last = band1 > band0 ? band1 - 1 : total - 1;

  // phase 1: every tile load in flight at once; out-of-band slots reload a valid
  // tile, which leaves the maximum unchanged and keeps the loads branch-free
  Raw8x8<T> raw[TPW];
  int tr[TPW], tc[TPW];
  bool ok[TPW];
#pragma unroll
  for (int k = 0; k < TPW; ++k) {
    const int t = band0 + lb + k * nx;
    ok[k] = t < band1;
    group_major_tile(ok[k] ? t : last, tiles_r, tiles_c, tr[k], tc[k]);
    nvfp4_tile_load<T>(x, tr[k] * 128, tc[k] * 128, rows, cols, raw[k]);
  }
  // The block maxima do not depend on the tensor scale: find them now, while the
  // loads and the exchange leave the ALUs idle, and park them in LDS for phase 2.
  __shared__ uint32_t bmw[TPW][kBlockMaxWords<T>][256];
  float m = 0.0f;
#pragma unroll
  for (int k = 0; k < TPW; ++k) {
    BlockMax<T> bm;
    bm.compute(raw[k]);
    m = __builtin_fmaxf(m, bm.lanemax());
    const uint32_t* w = reinterpret_cast<const uint32_t*>(&bm);
#pragma unroll
    for (int e = 0; e < kBlockMaxWords<T>; ++e) bmw[k][e][threadIdx.x] = w[e];
  }
  m = block_max256(m, gsh.red);
  const float g = grid_max<T>(ws, m, epoch, wait_iters, x, rows, cols, tiles_r, tiles_c, gsh);
  const float gs = tensor_scale_from_amax(g);
  if (b == 0 && threadIdx.x == 0) {
    *amax_out = g;
    *tensor_scale = gs;
  }

  // phase 2: quantize from registers
  fused_phase2<T, TPW, ROW, COL, SR, 0>(raw, bmw, tr, tc, ok, rows, cols, gs, stage, rtab, rcodes, rscales, ccodes,
                                        cscales, k0, k1);
}

namespace {

template <typename T, int TPW, bool ROW, bool COL, bool SR>
bool try_fused_t(const T* x, int rows, int cols, float* amax, float* ts, uint8_t* rc, uint8_t* rs, uint8_t* cc,
                 uint8_t* cs, uint32_t k0, uint32_t k1, FusedArea* area, uint32_t epoch, uint32_t wait_iters,
                 hipStream_t st) {
  const int tiles_r = (rows + 127) / 128, tiles_c = (cols + 127) / 128, total = tiles_r * tiles_c;
  const int per = (total + 7) / 8;
  const int nwg = 8 * ((per + TPW - 1) / TPW);
  auto kern = k_nvfp4_fused<T, TPW, ROW, COL, SR>;
  int per_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, 256, 0) != hipSuccess) return false;
  if (nwg > kFusedMaxWg || nwg > per_cu * num_cus()) return false;
  kern<<<nwg, 256, 0, st>>>(x, rows, cols, tiles_r, tiles_c, area, epoch, wait_iters, amax, ts, rc, rs, cc, cs, k0,
                            k1);
  return true;
}

template <typename T, bool ROW, bool COL, bool SR>
bool try_fused_rcs(const T* x, int rows, int cols, float* amax, float* ts, uint8_t* rc, uint8_t* rs, uint8_t* cc,
                   uint8_t* cs, uint32_t k0, uint32_t k1, FusedArea* area, uint32_t epoch, uint32_t wait_iters,
                   hipStream_t st) {
  // fewest tiles per workgroup that still fit one co-resident grid
#define FP4Q_TRY(N) try_fused_t<T, N, ROW, COL, SR>(x, rows, cols, amax, ts, rc, rs, cc, cs, k0, k1, area, epoch, \
                                                   wait_iters, st)
  if (FP4Q_TRY(1)) return true;
  if (FP4Q_TRY(2)) return true;
  if constexpr (sizeof(T) == 2)
    if (FP4Q_TRY(4)) return true;
#undef FP4Q_TRY
  return false;
}

template <typename T>
bool try_fused_dt(const void* xv, int64_t rows, int64_t cols, unsigned layouts, bool sr, float* amax, float* ts,
                  uint8_t* rc, uint8_t* rs, uint8_t* cc, uint8_t* cs, uint32_t k0, uint32_t k1, FusedArea* area,
                  uint32_t epoch, uint32_t wait_iters, hipStream_t st) {
  const T* x = static_cast<const T*>(xv);
  const bool row = layouts & 1u, col = layouts & 2u;
  const int r = (int)rows, c = (int)cols;
#define FP4Q_FU(R, C, S) \
  try_fused_rcs<T, R, C, S>(x, r, c, amax, ts, rc, rs, cc, cs, k0, k1, area, epoch, wait_iters, st)
  if (row && col) return sr ? FP4Q_FU(true, true, true) : FP4Q_FU(true, true, false);
  if (row) return sr ? FP4Q_FU(true, false, true) : FP4Q_FU(true, false, false);
  return sr ? FP4Q_FU(false, true, true) : FP4Q_FU(false, true, false);
#undef FP4Q_FU
}

}  // namespace

bool launch_nvfp4_fused(const void* x, int dtype, int64_t rows, int64_t cols, unsigned layouts, bool sr,
                        float* amax, float* tensor_scale, uint8_t* rc, uint8_t* rs, uint8_t* cc, uint8_t* cs,
                        uint64_t seed, FusedArea* area, uint32_t epoch, uint32_t wait_iters, hipStream_t st) {
  if (rows > (1 << 30) || cols > (1 << 30)) return false;
  const uint32_t k0 = (uint32_t)seed, k1 = (uint32_t)(seed >> 32);
  if (dtype == 1)
    return try_fused_dt<uint16_t>(x, rows, cols, layouts, sr, amax, tensor_scale, rc, rs, cc, cs, k0, k1, area, epoch,
                                  wait_iters, st);
  return try_fused_dt<float>(x, rows, cols, layouts, sr, amax, tensor_scale, rc, rs, cc, cs, k0, k1, area, epoch,
                             wait_iters, st);
}

// Zeroes n 32-bit words (a fill kernel rather than a memset, so it is also safe where
// a caller captures the stream).
__global__ __launch_bounds__(256) void k_fill_zero(uint32_t* __restrict__ p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) p[i] = 0u;
}

void launch_clear_scratch(void* p, int64_t bytes, hipStream_t st) {
  const int64_t n = bytes / 4;
  k_fill_zero<<<(int)((n + 255) / 256), 256, 0, st>>>(static_cast<uint32_t*>(p), n);
}

void launch_clear_fused(FusedArea* area, hipStream_t st) { launch_clear_scratch(area, sizeof(FusedArea), st); }

// ===========================================================================
// MXFP4: flat 1-D kernel over 4096 elements per workgroup.
//  RTN: load k (0..3) of wave w reads elements 1024w + 256k + 4l .. +3 into lane l, so
//  each load instruction covers 256 consecutive elements (whole cache lines, loaded
//  non-temporally); a 32-element block is eight consecutive lanes of one load, whose
//  maximum is three lane exchanges away (on fp32 8192 x 8192: 49 against 54 us for a
//  lane pair per block).
//  SR: a lane pair per block, each lane 16 consecutive elements, so that one Philox
//  call serves eight consecutive elements of one lane (the eight-lane layout would take
//  two calls per eight elements and is VALU-bound: 70 against 55 us).
// ===========================================================================

// AMAX: the workgroup also posts max|x| over its elements (magnitude bits compared as
// integers, so a NaN wins as it does in the amax pass) by atomic max into spread line
// b % kAmaxSpread of the workspace, which is zero when the call starts; k_spread_max
// folds the lines afterwards and clears them again.  Spreading the posts over
// kAmaxSpread cache lines keeps same-address atomics from queueing.  The post comes
// after the codes are stored.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t u) {
  u = max(u, (uint32_t)__builtin_amdgcn_mov_dpp((int)u, 0xB1, 0xF, 0xF, false));   // lane ^ 1
  u = max(u, (uint32_t)__builtin_amdgcn_mov_dpp((int)u, 0x4E, 0xF, 0xF, false));   // lane ^ 2
  u = max(u, (uint32_t)__builtin_amdgcn_mov_dpp((int)u, 0x141, 0xF, 0xF, false));  // the other quad of 8
  u = max(u, (uint32_t)__builtin_amdgcn_mov_dpp((int)u, 0x140, 0xF, 0xF, false));  // the other half of 16
  auto s16 = __builtin_amdgcn_permlane16_swap(u, u, false, false);                  // the other row of 32
  u = max(s16[0], s16[1]);
  auto s32 = __builtin_amdgcn_permlane32_swap(u, u, false, false);                  // the other half of 64
  return max(s32[0], s32[1]);
}

__device__ __forceinline__ void mx_post_amax(uint32_t mb, uint32_t* __restrict__ spread) {
  __shared__ uint32_t wm[4];
  mb = wave_max_u32(mb);
  if ((threadIdx.x & 63) == 0) wm[threadIdx.x >> 6] = mb;
  __syncthreads();
  if (threadIdx.x == 0)
    atomicMax(&spread[(blockIdx.x % kAmaxSpread) * 32], max(max(wm[0], wm[1]), max(wm[2], wm[3])));
}

template <typename T, bool SR, bool AMAX>
__global__ __launch_bounds__(256) void k_mxfp4(const T* __restrict__ x, int64_t n16,
                                               uint8_t* __restrict__ codes, uint8_t* __restrict__ scales,
                                               uint32_t k0, uint32_t k1, uint32_t* __restrict__ spread) {
  uint32_t mb = 0;   // max |x| magnitude bits over the lane's elements (AMAX)
  if constexpr (SR) {
    const int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x;   // 16-element group
    const bool ok = g < n16;
    float a[8], b[8];
    if (ok) {
      load8(x, g * 16, a);
      load8(x, g * 16 + 8, b);
    } else {
#pragma unroll
      for (int k = 0; k < 8; ++k) a[k] = b[k] = 0.0f;
    }
    float m = 0.0f;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      m = __builtin_fmaxf(m, __builtin_fmaxf(__builtin_fabsf(a[k]), __builtin_fabsf(b[k])));
      if constexpr (AMAX) mb = max(mb, max(__float_as_uint(a[k]) & 0x7FFFFFFFu, __float_as_uint(b[k]) & 0x7FFFFFFFu));
    }
    m = lane_xor_max<1>(m);
    const uint32_t code = e8m0_encode(__fdiv_rn(m, 6.0f));   // exact also for subnormal quotients
    // the converts use only the scale's exponent field: pass 2^(code-127) as its bits
    const float scale = __uint_as_float(code << 23);
    uint32_t ra[8], rb[8];
    sr_draws8((uint64_t)(g * 2), 0u, k0, k1, ra);
    sr_draws8((uint64_t)(g * 2 + 1), 0u, k0, k1, rb);
    const uint32_t w0 = pack8_sr(a, ra, scale), w1 = pack8_sr(b, rb, scale);
    if (ok) {
      *reinterpret_cast<uint2*>(codes + g * 8) = make_uint2(w0, w1);
      if ((threadIdx.x & 1) == 0) scales[g >> 1] = (uint8_t)code;
    }
  } else {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t n = n16 * 16;                              // a multiple of 32: blocks are whole
    const int64_t e0 = (int64_t)blockIdx.x * 4096 + wave * 1024 + 4 * lane;
    float v[4][4];
    bool ok[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int64_t e = e0 + 256 * k;
      ok[k] = e < n;                                         // the same for the block's 8 lanes
      load4(x + (ok[k] ? e : n - 4), v[k]);
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      float m = __builtin_fmaxf(__builtin_fmaxf(__builtin_fabsf(v[k][0]), __builtin_fabsf(v[k][1])),
                                __builtin_fmaxf(__builtin_fabsf(v[k][2]), __builtin_fabsf(v[k][3])));
      if constexpr (AMAX) {
        uint32_t mk = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) mk = max(mk, __float_as_uint(v[k][i]) & 0x7FFFFFFFu);
        mb = max(mb, ok[k] ? mk : 0u);
      }
      m = lane_xor_max<1>(m);
      m = lane_xor_max<2>(m);
      // the other quad of the eight lanes: row_half_mirror (lane i of 8 reads lane 7 - i)
      m = __builtin_fmaxf(m, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(m), 0x141, 0xF, 0xF, false)));
      const uint32_t code = e8m0_encode(__fdiv_rn(m, 6.0f));
      const float scale = __uint_as_float(code << 23);
      uint32_t w = __float_as_uint(v[k][0]);
      w = FP4Q_CVT_RTN(w, v[k][0], v[k][1], scale, 0);
      w = FP4Q_CVT_RTN(w, v[k][2], v[k][3], scale, 1);
      const int64_t e = e0 + 256 * k;
      if (ok[k]) {
        *reinterpret_cast<uint16_t*>(codes + (e >> 1)) = (uint16_t)w;
        if ((lane & 7) == 0) scales[e >> 5] = (uint8_t)code;
      }
    }
  }
  if constexpr (AMAX) mx_post_amax(mb, spread);
}

// The tensor amax from the spread lines; then every line is cleared for the next call
// (one workgroup: all reads are done before the barrier, all clears after it).
__global__ __launch_bounds__(256) void k_spread_max(uint32_t* __restrict__ spread, float* __restrict__ amax) {
  __shared__ uint32_t wm[4];
  uint32_t mb = 0;
  for (int i = threadIdx.x; i < kAmaxSpread; i += 256) mb = max(mb, spread[i * 32]);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) mb = max(mb, (uint32_t)__shfl_xor((int)mb, off, 64));
  if ((threadIdx.x & 63) == 0) wm[threadIdx.x >> 6] = mb;
  __syncthreads();
  for (int i = threadIdx.x; i < kAmaxSpread; i += 256) spread[i * 32] = 0u;
  if (threadIdx.x == 0) *amax = __uint_as_float(max(max(wm[0], wm[1]), max(wm[2], wm[3])));
}

void launch_mxfp4(const void* x, int dtype, int64_t rows, int64_t cols, bool sr, uint8_t* codes,
                  uint8_t* scales, uint64_t seed, float* amax, uint32_t* spread, hipStream_t st) {
  const int64_t n16 = rows * cols / 16;
  const int grid = (int)((n16 + 255) / 256);
  const uint32_t k0 = (uint32_t)seed, k1 = (uint32_t)(seed >> 32);
#define FP4Q_MX(TY, S, A) \
  k_mxfp4<TY, S, A><<<grid, 256, 0, st>>>(static_cast<const TY*>(x), n16, codes, scales, k0, k1, spread)
  if (dtype == 1) {
    if (amax) { if (sr) FP4Q_MX(uint16_t, true, true); else FP4Q_MX(uint16_t, false, true); }
    else      { if (sr) FP4Q_MX(uint16_t, true, false); else FP4Q_MX(uint16_t, false, false); }
  } else {
    if (amax) { if (sr) FP4Q_MX(float, true, true); else FP4Q_MX(float, false, true); }
    else      { if (sr) FP4Q_MX(float, true, false); else FP4Q_MX(float, false, false); }
  }
#undef FP4Q_MX
  if (amax) k_spread_max<<<1, 256, 0, st>>>(spread, amax);
}

// ===========================================================================
// IF4: flat kernel, one lane per 16-element row block (four blocks per lane).
// ===========================================================================

// Eight E2M1 nibbles -> values times 2^exponent(scale) (exact).
__device__ __forceinline__ void decode8_fp4(uint32_t w, float scale, float r[8]) {
  f32x2 d;
  d = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, scale, 0); r[0] = d[0]; r[1] = d[1];
  d = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, scale, 1); r[2] = d[0]; r[3] = d[1];
  d = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, scale, 2); r[4] = d[0]; r[5] = d[1];
  d = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, scale, 3); r[6] = d[0]; r[7] = d[1];
}

// INT4 candidate for 8 scaled values under the 6/7 rule: q = clamp(rint(v*fl(7/6)), -7, 7)
// via the 1.5*2^23 rounding constant (its low nibble is q in two's complement), restored
// as fl(q*fl(6/7)); accumulates both squared-error sums in element order.
// The clamp only matters in blocks whose E4M3 scale is subnormal: with a normal scale s
// (code >= 8) the scale is at least 15/16 of fl(bamax*gs)/6, so |v| <= 6.4 (one ulp
// more at most) and |fl(v*fl(7/6))| <= 7.47, which rounds to at most 7 anyway.
// The restore fl(q*fl(6/7)) comes from a 16-entry LDS table indexed by q + 8, whose
// byte address is one shift-and-add of y's bits (y = 1.5*2^23 + q as an integer).
struct If4RestoreTable {
  float r[16];   // r[i] = fl((i - 8) * fl(6/7))
};
constexpr uint32_t kIf4MagicBits = 0x4B400000u;   // bits of 1.5*2^23

__device__ __forceinline__ void fill_if4_restore(If4RestoreTable& t) {
  if (threadIdx.x < 16) t.r[threadIdx.x] = (float)((int)threadIdx.x - 8) * (6.0f / 7.0f);
}

template <bool CLAMP>
__device__ __forceinline__ uint32_t if4_block8(const float v[8], const float rf[8], const If4RestoreTable& rt,
                                               float& e_fp, float& e_int) {
  const float c76 = 7.0f / 6.0f, magic = 12582912.0f;
  // &rt.r[q + 8] = rt.r + (bits(y) - kIf4MagicBits + 8), all in 32-bit LDS addresses
  const float* base = rt.r + 8 - kIf4MagicBits;
  uint32_t yb[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    float wv = v[k] * c76;
    if constexpr (CLAMP) wv = __builtin_amdgcn_fmed3f(wv, -7.0f, 7.0f);
    const float y = wv + magic;
    yb[k] = __float_as_uint(y);
    const float ri = base[yb[k]];
    const float dfp = v[k] - rf[k];
    const float dint = v[k] - ri;
    e_fp = __builtin_fmaf(dfp, dfp, e_fp);
    e_int = __builtin_fmaf(dint, dint, e_int);
  }
  // nibble k = low nibble of yb[k]: gather the low bytes of the even and the odd
  // elements (byte permutes), then merge the two nibble planes in one bit select
  const uint32_t ev = __builtin_amdgcn_perm(yb[2], yb[0], 0x0C0C0400u) | __builtin_amdgcn_perm(yb[6], yb[4], 0x04000C0Cu);
  const uint32_t od = __builtin_amdgcn_perm(yb[3], yb[1], 0x0C0C0400u) | __builtin_amdgcn_perm(yb[7], yb[5], 0x04000C0Cu);
  return __builtin_amdgcn_bitop3_b32(ev, od << 4, 0x0F0F0F0Fu, 0xE4);   // (ev & m) | (od<<4 & ~m)
}

// Each lane takes kIf4Blocks blocks, one from each of the workgroup's consecutive
// 256-block chunks (so every load instruction stays contiguous across the wave); all
// their loads are issued before any block is encoded, and the per-launch work (tensor
// scale, reciprocal table) is shared by the four.
constexpr int kIf4Blocks = 4;

// One 16-element block held as two halves a, b of scaled values x*gs: scale, both
// candidates, choice.  Writes the 8 code bytes and the flagged scale byte.
template <bool CLAMP>
__device__ __forceinline__ void if4_encode(float (&a)[8], float (&b)[8], uint32_t sc, const RecipPair rp,
                                           const If4RestoreTable& rt, uint2& codes, uint32_t& scale) {
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    a[k] = div2(a[k], rp);
    b[k] = div2(b[k], rp);
  }
  const uint32_t fa = pack8_rtn(a, 1.0f), fb = pack8_rtn(b, 1.0f);
  float ra[8], rb[8];
  decode8_fp4(fa, 1.0f, ra);
  decode8_fp4(fb, 1.0f, rb);
  float e_fp = 0.0f, e_int = 0.0f;
  const uint32_t ia = if4_block8<CLAMP>(a, ra, rt, e_fp, e_int);
  const uint32_t ib = if4_block8<CLAMP>(b, rb, rt, e_fp, e_int);
  const bool use_int = e_int < e_fp;
  codes = use_int ? make_uint2(ia, ib) : make_uint2(fa, fb);
  scale = sc | (use_int ? 0x80u : 0u);
}

// max |v| over 16 values, as a tree of three-input maxima.
__device__ __forceinline__ float absmax16(const float (&a)[8], const float (&b)[8]) {
  auto m3 = [](float x, float y, float z) {
    return __builtin_fmaxf(__builtin_fmaxf(__builtin_fabsf(x), __builtin_fabsf(y)), __builtin_fabsf(z));
  };
  const float p0 = m3(a[0], a[1], a[2]), p1 = m3(a[3], a[4], a[5]), p2 = m3(a[6], a[7], b[0]);
  const float p3 = m3(b[1], b[2], b[3]), p4 = m3(b[4], b[5], b[6]);
  return __builtin_fmaxf(__builtin_fmaxf(__builtin_fmaxf(p0, p1), p2),
                         __builtin_fmaxf(__builtin_fmaxf(p3, p4), __builtin_fabsf(b[7])));
}

// The blocks of one lane.  CHECK: the workgroup's last chunk may run past n16 (loads
// are clamped to the last block and stores skipped); otherwise every block exists.
template <typename T, bool CHECK>
__device__ __forceinline__ void if4_lane(const T* __restrict__ x, int64_t n16, float gs, const RecipTable& rtab,
                                         const If4RestoreTable& rt, uint8_t* __restrict__ codes,
                                         uint8_t* __restrict__ scales) {
  const int64_t g0 = (int64_t)blockIdx.x * (256 * kIf4Blocks) + threadIdx.x;
  float a[kIf4Blocks][8], b[kIf4Blocks][8];
#pragma unroll
  for (int j = 0; j < kIf4Blocks; ++j) {
    const int64_t g = CHECK ? min(g0 + 256 * j, n16 - 1) : g0 + 256 * j;
    load8(x, g * 16, a[j]);
    load8(x, g * 16 + 8, b[j]);
  }
#pragma unroll
  for (int j = 0; j < kIf4Blocks; ++j) {
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      a[j][k] = a[j][k] * gs;
      b[j][k] = b[j][k] * gs;
    }
    const uint32_t sc = nvfp4_scale_code(absmax16(a[j], b[j]));
    const RecipPair rp = rtab.r[sc];
    uint2 cw;
    uint32_t sw;
    // the clamp only for waves holding a block with a subnormal scale (uniform branch)
    if (__builtin_amdgcn_ballot_w64(sc < 8u) != 0)
      if4_encode<true>(a[j], b[j], sc, rp, rt, cw, sw);
    else
      if4_encode<false>(a[j], b[j], sc, rp, rt, cw, sw);
    const int64_t g = g0 + 256 * j;
    if (!CHECK || g < n16) {
      *reinterpret_cast<uint2*>(codes + g * 8) = cw;
      scales[g] = (uint8_t)sw;
    }
  }
}

template <typename T>
__global__ __launch_bounds__(256) void k_if4(const T* __restrict__ x, int64_t n16, AmaxSource amax,
                                             float* __restrict__ tensor_scale, uint8_t* __restrict__ codes,
                                             uint8_t* __restrict__ scales) {
  __shared__ RecipTable rtab;
  __shared__ If4RestoreTable rt;
  fill_recip_table(rtab);
  fill_if4_restore(rt);
  __syncthreads();
  const float gs = tensor_scale_publish(amax, tensor_scale);
  if ((int64_t)(blockIdx.x + 1) * (256 * kIf4Blocks) <= n16)
    if4_lane<T, false>(x, n16, gs, rtab, rt, codes, scales);
  else
    if4_lane<T, true>(x, n16, gs, rtab, rt, codes, scales);
}

void launch_if4(const void* x, int dtype, int64_t rows, int64_t cols, const AmaxSource& amax, float* tensor_scale,
                uint8_t* codes, uint8_t* scales, hipStream_t st) {
  const int64_t n16 = rows * cols / 16;
  const int grid = (int)((n16 + 256 * kIf4Blocks - 1) / (256 * kIf4Blocks));
  if (dtype == 1)
    k_if4<uint16_t><<<grid, 256, 0, st>>>(static_cast<const uint16_t*>(x), n16, amax, tensor_scale, codes, scales);
  else
    k_if4<float><<<grid, 256, 0, st>>>(static_cast<const float*>(x), n16, amax, tensor_scale, codes, scales);
}

// ===========================================================================
// NVFP4 16x16 (2D).  Sixteen lanes own one 16x16 tile, four columns of four rows
// each; a wave holds four horizontally adjacent tiles.  The tile maximum is a
// 16-lane reduction.  The optional transposed codes go through LDS.
// ===========================================================================

// Maximum over the 16 lanes of one 16x16 tile in the layout of k_nvfp4_2d: lanes
// l ^ 1, l ^ 2 (DPP within the quad), l ^ 16 and l ^ 32 (lane-row swaps).
__device__ __forceinline__ float max_tile_lanes(float v) {
  v = lane_xor_max<1>(v);
  v = lane_xor_max<2>(v);
  const uint32_t u = __float_as_uint(v);
  auto s16 = __builtin_amdgcn_permlane16_swap(u, u, false, false);   // (own, l ^ 16) in some order
  const float m16 = __builtin_fmaxf(__uint_as_float(s16[0]), __uint_as_float(s16[1]));
  const uint32_t w = __float_as_uint(m16);
  auto s32 = __builtin_amdgcn_permlane32_swap(w, w, false, false);   // (own, l ^ 32) in some order
  return __builtin_fmaxf(__uint_as_float(s32[0]), __uint_as_float(s32[1]));
}

// A wave holds four horizontally adjacent 16x16 tiles per run.  Lane l = 16q + 4t + u
// takes columns 4u..4u+3 of tile t in rows q, q+4, q+8 and q+12, so each of its four
// row loads is one instruction over four whole 64-column row pieces (one contiguous
// 256-byte span per row in a 16-aligned run of tiles).  A workgroup takes k2dSteps
// consecutive runs of 16 tiles; all of a lane's row loads are issued before any tile
// is encoded.  Each lane stores the 2 code bytes of its four columns per row: one
// store instruction writes four rows' 32 contiguous bytes per tile run of a wave.
constexpr int k2dSteps = 4;

template <typename T, bool TRANS>
__global__ __launch_bounds__(256) void k_nvfp4_2d(const T* __restrict__ x, int64_t rows, int64_t cols,
                                                  AmaxSource amax, float* __restrict__ tensor_scale,
                                                  uint8_t* __restrict__ codes, uint8_t* __restrict__ scales,
                                                  uint8_t* __restrict__ codes_t) {
  __shared__ uint32_t lds[k2dSteps][16][16][2];   // [run][tile in run][row][8 bytes]
  __shared__ RecipTable rtab;
  fill_recip_table(rtab);
  __syncthreads();
  const float gs = tensor_scale_publish(amax, tensor_scale);
  const int64_t tiles_c = cols >> 4, tiles = (rows >> 4) * tiles_c;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int q = lane >> 4, tin = (lane >> 2) & 3, u = lane & 3;
  float v[k2dSteps][16];   // v[j][4k + e]: row q + 4k, column 4u + e of the lane's tile
  int64_t br[k2dSteps], bc[k2dSteps];
  bool ok[k2dSteps];
#pragma unroll
  for (int j = 0; j < k2dSteps; ++j) {
    const int64_t tile = ((int64_t)blockIdx.x * k2dSteps + j) * 16 + wave * 4 + tin;
    ok[j] = tile < tiles;
    const int64_t t = ok[j] ? tile : tiles - 1;            // past the end: reload the last tile
    br[j] = t / tiles_c;
    bc[j] = t - br[j] * tiles_c;
    const T* px = x + (br[j] * 16 + q) * cols + bc[j] * 16 + 4 * u;
#pragma unroll
    for (int k = 0; k < 4; ++k) load4(px + 4 * k * cols, &v[j][4 * k]);
  }
#pragma unroll
  for (int j = 0; j < k2dSteps; ++j) {
    float m = 0.0f;
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      v[j][k] = v[j][k] * gs;
      m = __builtin_fmaxf(m, __builtin_fabsf(v[j][k]));
    }
    m = max_tile_lanes(m);
    const uint32_t sc = nvfp4_scale_code(m);
    const RecipPair rp = rtab.r[sc];
#pragma unroll
    for (int k = 0; k < 16; ++k) v[j][k] = div2(v[j][k], rp);
    // w0: rows q (bits 0..15) and q + 4 (16..31); w1: rows q + 8 and q + 12
    const uint32_t w0 = pack8_rtn(&v[j][0], 1.0f), w1 = pack8_rtn(&v[j][8], 1.0f);
    const uint16_t piece[4] = {(uint16_t)w0, (uint16_t)(w0 >> 16), (uint16_t)w1, (uint16_t)(w1 >> 16)};
    if (ok[j]) {
      uint8_t* dst = codes + (br[j] * 16 + q) * (cols >> 1) + bc[j] * 8 + 2 * u;
#pragma unroll
      for (int k = 0; k < 4; ++k) *reinterpret_cast<uint16_t*>(dst + 4 * k * (cols >> 1)) = piece[k];
      if ((lane & 0x33) == 0) scales[br[j] * tiles_c + bc[j]] = (uint8_t)sc;   // q == 0, u == 0
    }
    if constexpr (TRANS) {
      uint16_t* l16 = reinterpret_cast<uint16_t*>(&lds[j][wave * 4 + tin][0][0]);
#pragma unroll
      for (int k = 0; k < 4; ++k) l16[(q + 4 * k) * 4 + u] = piece[k];
    }
  }
  if constexpr (TRANS) {
    __syncthreads();
    // lane l now gathers column i = l & 15 of tile l >> 4 of its wave: nibble i of every row
    const int tt = lane >> 4, i = lane & 15;
    const int tb = wave * 4 + tt, word = i >> 3, sh = (i & 7) * 4;
#pragma unroll
    for (int j = 0; j < k2dSteps; ++j) {
      uint32_t o0 = 0, o1 = 0;
#pragma unroll
      for (int rr = 0; rr < 8; ++rr) {
        o0 |= ((lds[j][tb][rr][word] >> sh) & 0xFu) << (4 * rr);
        o1 |= ((lds[j][tb][rr + 8][word] >> sh) & 0xFu) << (4 * rr);
      }
      const int64_t tile = ((int64_t)blockIdx.x * k2dSteps + j) * 16 + tb;
      if (tile < tiles) {
        const int64_t tr = tile / tiles_c, tc = tile - tr * tiles_c;
        *reinterpret_cast<uint2*>(codes_t + (tc * 16 + i) * (rows >> 1) + (tr * 16 >> 1)) = make_uint2(o0, o1);
      }
    }
  }
}

void launch_nvfp4_2d(const void* x, int dtype, int64_t rows, int64_t cols, const AmaxSource& amax, float* tensor_scale,
                     uint8_t* codes, uint8_t* scales, uint8_t* codes_t, hipStream_t st) {
  const int64_t tiles = (rows >> 4) * (cols >> 4);
  const int grid = (int)((tiles + 16 * k2dSteps - 1) / (16 * k2dSteps));
#define FP4Q_2D(T, TR) k_nvfp4_2d<T, TR><<<grid, 256, 0, st>>>(static_cast<const T*>(x), rows, cols, amax, \
                                                              tensor_scale, codes, scales, codes_t)
  if (dtype == 1) { if (codes_t) FP4Q_2D(uint16_t, true); else FP4Q_2D(uint16_t, false); }
  else            { if (codes_t) FP4Q_2D(float, true); else FP4Q_2D(float, false); }
#undef FP4Q_2D
}

// ===========================================================================
// Dequantize: x_hat = fl(fl(r*s)/gs) (NVFP4, 2D, IF4) or r*2^(code-127) (MXFP4).
// The lanes of a wave write consecutive 16-byte chunks, so each store instruction
// covers one contiguous span of 1 KiB; a lane handles 16 elements of a 1024-element
// wave span, in four steps of four fp32 outputs or two steps of eight bf16 outputs.
// The output is written once and whole lines at a time, so its stores (and the code
// loads of the bf16 form) are non-temporal: on the IF4 round trip of bf16
// 32768 x 8192 the dequantization takes 107 instead of 113 us, and the quantization
// that follows it in the next step finds the caches free (whole step 339 -> 316 us).
// ===========================================================================

// Two fp32 values -> packed bf16 (first in the low half), round to nearest even: one
// v_cvt_pk_bf16_f32 (gfx950).
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2_t));
}

template <int FMT, bool BF16OUT>
__global__ __launch_bounds__(256) void k_dequant(const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales,
                                                 const float* __restrict__ tensor_scale, int64_t rows, int64_t cols,
                                                 void* __restrict__ y) {
  constexpr int EPL = BF16OUT ? 8 : 4;          // elements per lane and step
  constexpr int STEPS = 16 / EPL;
  const int lane = threadIdx.x & 63;
  const int64_t n = rows * cols;                // a multiple of 16
  const int64_t e0 = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * 1024 + lane * EPL;
  if (e0 >= n) return;

  // loads first, from clamped addresses, so all of them are in flight together
  uint32_t cw[STEPS], sc[STEPS];
  int64_t r = 0, c = 0;
  if constexpr (FMT == 1) { r = e0 / cols; c = e0 - r * cols; }
#pragma unroll
  for (int j = 0; j < STEPS; ++j) {
    const int64_t e = min(e0 + (int64_t)j * 64 * EPL, n - EPL);
    if constexpr (EPL == 4) cw[j] = *reinterpret_cast<const uint16_t*>(codes + (e >> 1));
    else cw[j] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(codes + (e >> 1)));
    if constexpr (FMT == 2) {
      sc[j] = scales[e >> 5];
    } else if constexpr (FMT == 1) {
      const int64_t rr = min(r, rows - 1);
      sc[j] = scales[(rr >> 4) * (cols >> 4) + (c >> 4)];
      c += 64 * EPL;
      while (c >= cols) { c -= cols; ++r; }
    } else {
      sc[j] = scales[e >> 4];
    }
  }
  float gs = 1.0f, rgs = 1.0f;
  if constexpr (FMT != 2) { gs = *tensor_scale; rgs = __fdiv_rn(1.0f, gs); }

#pragma unroll
  for (int j = 0; j < STEPS; ++j) {
    const int64_t e = e0 + (int64_t)j * 64 * EPL;
    if (e >= n) break;
    float rv[EPL], out[EPL];
    if (FMT == 4 || (FMT == 3 && (sc[j] & 0x80u))) {
      // INT4 restore: fl(q * fl(6/7)) for IF4's flagged blocks, q itself for NVINT4 (FMT 4)
      const float c = FMT == 4 ? 1.0f : 6.0f / 7.0f;
#pragma unroll
      for (int k = 0; k < EPL; ++k) rv[k] = (float)((int)(((cw[j] >> (4 * k)) & 0xFu) ^ 8u) - 8) * c;
    } else {
      f32x2 d = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cw[j], 1.0f, 0);
      rv[0] = d[0]; rv[1] = d[1];
      d = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cw[j], 1.0f, 1);
      rv[2] = d[0]; rv[3] = d[1];
      if constexpr (EPL == 8) {
        d = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cw[j], 1.0f, 2);
        rv[4] = d[0]; rv[5] = d[1];
        d = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cw[j], 1.0f, 3);
        rv[6] = d[0]; rv[7] = d[1];
      }
    }
    if constexpr (FMT == 2) {
      // E8M0: exact power-of-two scaling, subnormal and overflowing results included
#pragma unroll
      for (int k = 0; k < EPL; ++k) out[k] = __builtin_ldexpf(rv[k], (int)sc[j] - 127);
    } else {
      // fl(t/gs) for t = fl(r*s): over all element and scale codes t has only 29
      // significands, and for each of them the corrected-reciprocal division is
      // correctly rounded against every divisor significand (checked exhaustively on
      // the host).  That carries over to every exponent while no intermediate leaves
      // the normal range, which s/gs in [2^-98, 2^96] (with |r| in [0.5, 48/7])
      // guarantees; other blocks, and non-finite or negative scales, divide exactly.
      const float s = e4m3_decode(sc[j] & 0x7Fu);
      const float ratio = s * rgs;
      if (ratio >= 0x1p-98f && ratio <= 0x1p+96f) {
#pragma unroll
        for (int k = 0; k < EPL; ++k) out[k] = div_rs(rv[k] * s, gs, rgs);
      } else {
#pragma unroll
        for (int k = 0; k < EPL; ++k) out[k] = __fdiv_rn(rv[k] * s, gs);
      }
    }
    if constexpr (BF16OUT) {
      uint4 o;
      o.x = pack_bf16x2(out[0], out[1]);
      o.y = pack_bf16x2(out[2], out[3]);
      o.z = pack_bf16x2(out[4], out[5]);
      o.w = pack_bf16x2(out[6], out[7]);
      __builtin_nontemporal_store(u32x4_t{o.x, o.y, o.z, o.w}, reinterpret_cast<u32x4_t*>(static_cast<uint16_t*>(y) + e));
    } else {
      __builtin_nontemporal_store(f32x4_t{out[0], out[1], out[2], out[3]}, reinterpret_cast<f32x4_t*>(static_cast<float*>(y) + e));
    }
  }
}

void launch_dequant(int fmt, const uint8_t* codes, const uint8_t* scales, const float* tensor_scale, int64_t rows,
                    int64_t cols, int out_dtype, void* y, hipStream_t st) {
  const int64_t n = rows * cols;
  const int grid = (int)((n + 4095) / 4096);
#define FP4Q_DQ(F) \
  if (out_dtype == 1) k_dequant<F, true><<<grid, 256, 0, st>>>(codes, scales, tensor_scale, rows, cols, y); \
  else k_dequant<F, false><<<grid, 256, 0, st>>>(codes, scales, tensor_scale, rows, cols, y)
  switch (fmt) {
    case 0: FP4Q_DQ(0); break;
    case 1: FP4Q_DQ(1); break;
    case 2: FP4Q_DQ(2); break;
    case 3: FP4Q_DQ(3); break;
    default: FP4Q_DQ(4); break;   // NVINT4 (the block-format variant), not a public format code
  }
#undef FP4Q_DQ
}

// ---------------------------------------------------------------------------------------
// MX FP6 (blog.ast.moe "FP6から考えるLLM量子化", sections "FP6で隣り合う値の間隔を見てみる"
// and "量子化と6bitの保存"): E2M3 (FMT 0: bias 1, largest 7.5) or E3M2 (FMT 1: bias 3,
// largest 28), subnormals at exponent 0, no Inf or NaN; 32-element blocks with an E8M0
// scale as MXFP4; four codes per three bytes, code j of a group in bits 6j .. 6j+5 of the
// little-endian 24-bit word, so a lane's 16 codes are one 96-bit little-endian word.
// ---------------------------------------------------------------------------------------

// One lane per 16 elements, a lane pair per block (as k_mxfp4).
template <typename T, int FMT>
__global__ __launch_bounds__(256) void k_mxfp6(const T* __restrict__ x, int64_t n16, uint8_t* __restrict__ codes,
                                               uint8_t* __restrict__ scales) {
  __shared__ uint32_t stg[4][sizeof(T) * 256];   // each wave's span: 4 KB (fp32) or 2 KB (bf16)
  const int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const bool ok = g < n16;
  float a[16];
  uint32_t* buf = stg[threadIdx.x >> 6];
  stage_issue16(x, n16 * 16, ((int64_t)blockIdx.x * 256 + (threadIdx.x & ~63u)) * 16, buf);
  stage_wait();
  stage_read16<T>(buf, a);
  if (!ok) {
#pragma unroll
    for (int k = 0; k < 16; ++k) a[k] = 0.0f;
  }
  float m = 0.0f;
#pragma unroll
  for (int k = 0; k < 16; ++k) m = __builtin_fmaxf(m, __builtin_fabsf(a[k]));
  m = lane_xor_max<1>(m);
  const uint32_t code = e8m0_encode(__fdiv_rn(m, FMT ? 28.0f : 7.5f));
  const float inv = e8m0_value(254u - code);   // 2^(127 - code), exact
#pragma unroll
  for (int k = 0; k < 16; ++k) a[k] *= inv;
  // one convert for the lane's 16 elements (given twice; the second copy is not used)
  const u32x6v cw = fp6_encode32<FMT>(a, a);
  const uint32_t w0 = cw[0], w1 = cw[1], w2 = cw[2];
  if (ok) {
    uint32_t* dst = reinterpret_cast<uint32_t*>(codes + g * 12);
    dst[0] = w0;
    dst[1] = w1;
    dst[2] = w2;
    if ((threadIdx.x & 1) == 0) scales[g >> 1] = (uint8_t)code;
  }
}

template <int FMT, bool BF16OUT>
__global__ __launch_bounds__(256) void k_dequant_mxfp6(const uint8_t* __restrict__ codes,
                                                       const uint8_t* __restrict__ scales, int64_t n16,
                                                       void* __restrict__ y) {
  const int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (g >= n16) return;
  const uint32_t* src = reinterpret_cast<const uint32_t*>(codes + g * 12);
  const float s = e8m0_value(scales[g >> 1]);
  u32x6v cw;
  cw[0] = src[0];
  cw[1] = src[1];
  cw[2] = src[2];
  cw[3] = cw[0];
  cw[4] = cw[1];
  cw[5] = cw[2];
  const f32x32v r = fp6_decode32<FMT>(cw);   // elements 16..31 repeat 0..15
  float v[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) v[i] = r[i] * s;
  if constexpr (BF16OUT) {
    uint32_t o[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) o[i] = pack_bf16x2(v[2 * i], v[2 * i + 1]);
    uint4* d = reinterpret_cast<uint4*>(static_cast<uint16_t*>(y) + g * 16);
    d[0] = make_uint4(o[0], o[1], o[2], o[3]);
    d[1] = make_uint4(o[4], o[5], o[6], o[7]);
  } else {
    float4* d = reinterpret_cast<float4*>(static_cast<float*>(y) + g * 16);
#pragma unroll
    for (int q = 0; q < 4; ++q) d[q] = make_float4(v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]);
  }
}

void launch_mxfp6(const void* x, int dtype, int64_t rows, int64_t cols, int fmt, uint8_t* codes, uint8_t* scales,
                  hipStream_t st) {
  const int64_t n16 = rows * cols / 16;
  const int grid = (int)((n16 + 255) / 256);
  if (dtype == 1) {
    if (fmt) k_mxfp6<uint16_t, 1><<<grid, 256, 0, st>>>(static_cast<const uint16_t*>(x), n16, codes, scales);
    else k_mxfp6<uint16_t, 0><<<grid, 256, 0, st>>>(static_cast<const uint16_t*>(x), n16, codes, scales);
  } else {
    if (fmt) k_mxfp6<float, 1><<<grid, 256, 0, st>>>(static_cast<const float*>(x), n16, codes, scales);
    else k_mxfp6<float, 0><<<grid, 256, 0, st>>>(static_cast<const float*>(x), n16, codes, scales);
  }
}

void launch_dequant_mxfp6(int fmt, const uint8_t* codes, const uint8_t* scales, int64_t rows, int64_t cols,
                          int out_dtype, void* y, hipStream_t st) {
  const int64_t n16 = rows * cols / 16;
  const int grid = (int)((n16 + 255) / 256);
  auto kern = fmt ? (out_dtype == 1 ? k_dequant_mxfp6<1, true> : k_dequant_mxfp6<1, false>)
                  : (out_dtype == 1 ? k_dequant_mxfp6<0, true> : k_dequant_mxfp6<0, false>);
  kern<<<grid, 256, 0, st>>>(codes, scales, n16, y);
}

}  // namespace fp4q

