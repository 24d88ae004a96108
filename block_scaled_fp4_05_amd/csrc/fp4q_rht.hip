// fp4q_rht.hip -- 128x128 random Hadamard transform along the token (row) dimension,
// qiita.com/nishiha/items/b98c2b931d588c4c81d5, section "ランダムアダマール変換": the
// Wgrad operands are multiplied by H (H H^T = I after 1/sqrt(128) scaling) whose
// rows are randomised by a +-1 diagonal S.  Per chunk of 128 rows:
//   B = R^T A,  R = S H / sqrt(128),  B[i][j] = sum_t H[i][t] s_t A[t][j] / sqrt(128).
//
// bf16 inputs run the contraction on MFMA (v_mfma_f32_32x32x16_bf16): the +-1
// matrix K[i][t] = H[i][t] s_t is exact in bf16 and the sum is accumulated in fp32.
// One wave owns a tile of 128 tokens x 64 columns.  The B operands (8 consecutive
// tokens of one column per lane) come either from registers -- the standalone
// transform loads a 2-column x 64-token slice per lane with 4-byte loads and pairs
// the tokens with v_perm -- or, in the fused passes, from the tile staged in LDS by
// direct loads and read back with transposing LDS reads (ds_read_b64_tr_b16).
// Sylvester H factors as H_128[32a+u][32b+w] = H_4[a][b] H_32[u][w]: the A operand of
// a K-step only depends on the H_32 part (folded with the signs, kept in registers for
// the wave's lifetime, with a negated copy), and the H_4 sign picks the negated A
// operand for the output row-blocks that need it.
//
// The standalone transform, the amax pass and the fused column-wise NVFP4 pass issue
// the same MFMA sequence for every output element (only the column's MFMA slot
// differs), so all three see bitwise identical values B = fl(acc * fl(1/sqrt(128))).
#include "fp4q_dev.hpp"
#include "fp4q_internal.hpp"

namespace fp4q {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr float kRhtScale = 0.08838834764831845f;   // fl(1/sqrt(128))

struct RhtSigns { uint32_t w[4]; };

__device__ __forceinline__ uint32_t parity(uint32_t v) { return __builtin_popcount(v) & 1u; }

// A-operand fragments: lane (il = lane & 31, hk = lane >> 5), K-step kk holds
// K[32a + il][16kk + 8hk + e] without the H_4 factor, e = 0..7.  Where H_4 is -1 the
// MFMA takes the fragment with its eight sign bits flipped (four XORs), made at the
// point of use rather than kept in registers.
__device__ __forceinline__ void make_fragments(const RhtSigns& sg, bool with_signs, u32x4 frag[8]) {
  const uint32_t lane = threadIdx.x & 63, il = lane & 31, hk = lane >> 5;
#pragma unroll
  for (int kk = 0; kk < 8; ++kk) {
    uint32_t d[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      uint32_t half[2];
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        const uint32_t t = 16u * kk + 8u * hk + 2u * q + b;      // token within the chunk
        uint32_t neg = parity(il & (t & 31u));
        if (with_signs) neg ^= (sg.w[t >> 5] >> (t & 31u)) & 1u;
        half[b] = 0x3F80u | (neg << 15);                          // bf16 +-1
      }
      d[q] = half[0] | (half[1] << 16);
    }
    frag[kk] = u32x4{d[0], d[1], d[2], d[3]};
  }
}

// The A operand of K-step kk for output block a: frag[kk] times H_4[a][kk/2] (a and kk
// are constants after unrolling, so the choice costs nothing).
__device__ __forceinline__ bf16x8 a_operand(const u32x4 frag[8], int a, int kk) {
  const bool flip = (__builtin_popcount(a & (kk >> 1)) & 1) != 0;
  return __builtin_bit_cast(bf16x8, flip ? (frag[kk] ^ 0x80008000u) : frag[kk]);
}

// The 64 words one lane reads for a tile: tokens tok0 + 16kk + 8hk + r (r = 0..7) of
// columns colp, colp+1.  All loads are issued before any MFMA and none sits under a
// branch, so the tile costs one memory round trip: a lane past the last column reads
// column pair 0 instead and its results are discarded by the caller.
struct RhtRaw {
  uint32_t v[8][8];
};

__device__ __forceinline__ void rht_load(const uint16_t* __restrict__ x, int64_t cols, int64_t tok0, int64_t colp,
                                         bool valid, RhtRaw& raw) {
  const uint32_t hk = (threadIdx.x & 63) >> 5;
  const uint16_t* base = x + (tok0 + 8 * hk) * cols + (valid ? colp : 0);
#pragma unroll
  for (int kk = 0; kk < 8; ++kk)
#pragma unroll
    for (int r = 0; r < 8; ++r)
      raw.v[kk][r] = *reinterpret_cast<const uint32_t*>(base + (int64_t)(16 * kk + r) * cols);
}

// LDS staging for the fused passes.  A wave's tile (128 tokens x 64 columns of bf16,
// 16 KB) goes from HBM to its own LDS buffer by 16 direct loads of 16 bytes per lane:
// lane l of load i lands at byte 16 l of that load's 1 KB, i.e. at token row
// r = 8i + l/8, chunk position l%8 of the row's 128 bytes, and it carries the row's
// column chunk (l%8) ^ swz(r) (8 columns).  No VGPR holds the data in flight, so a
// wave keeps a whole tile in the air while it works on the previous one, and two
// waves fit on each SIMD.  Chunks past the last column read column chunk 0 of the same
// token instead; only lanes whose results are discarded use them.
struct RhtStage {
  uint32_t w[128 * 32];
};

// Chunk swizzle of staged row r: it depends on r % 4 only, and it spreads the
// transposed reads below over distinct LDS banks (with 32 or 64 banks).
__device__ __forceinline__ uint32_t rht_swz(uint32_t r) { return ((r & 1u) * 3u) | (((r >> 1) & 1u) << 2); }

// The address of load i is the uniform row base of tokens tok0 + 8i (scalar registers)
// plus this lane's byte offset, which fits 32 bits because cols < 2^27 (checked by the
// caller); with the buffer picked by a uniform wave index, the per-load address and
// LDS base steps run on the scalar unit.  NT marks the loads non-temporal: the
// quantizer's read is the operand's last, and with it the amax pass of the next
// operand runs 26 instead of 30 us on bf16 16384 x 4096 (the quantizer itself is as
// fast either way); the amax pass keeps normal loads, which leave the operand in the
// Infinity Cache for the quantizer after it.
template <bool NT>
__device__ __forceinline__ void rht_issue(const uint16_t* __restrict__ x, int64_t cols, int64_t tok0, int64_t col0,
                                          RhtStage& st) {
  const uint32_t lane = threadIdx.x & 63;
  const int64_t c = col0 + 8 * ((lane & 7) ^ rht_swz((lane >> 3) & 3));
  const uint32_t off = 2u * ((lane >> 3) * (uint32_t)cols + (uint32_t)(c < cols ? c : 0));
  const char* rows0 = reinterpret_cast<const char*>(x + tok0 * cols);
#pragma unroll
  for (int i = 0; i < 16; ++i)
    __builtin_amdgcn_global_load_lds(rows0 + (int64_t)(16 * i) * cols + off, &st.w[i * 256], 16, 0, NT ? 2 : 0);   // aux bit 1: nt
}

// The direct loads are invisible to the compiler's wait counting: wait for every
// outstanding vector memory operation before the buffer is read, and for the LDS
// reads before it is refilled.
__device__ __forceinline__ void rht_wait_loads() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
__device__ __forceinline__ void rht_wait_lds() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// MFMA B operands of a staged tile, read transposed from LDS.  In the fused passes
// MFMA column slot n of pass p is tile column 32p + n.  The B operand of K-step kk
// holds, in lane (n, hk), tokens 16kk + 8hk + 0..7 of that column, two per dword.
// ds_read_b64_tr_b16 hands output lane i of each 16-lane group element i%4 of the
// 8-byte reads of source lanes i/4 + 4e (e = 0..3, one 16-bit element per e), so
// source lane 4e + a reads token k0 + e, columns c0 + 4a..4a+3, and output lane i
// receives tokens k0..k0+3 of column c0 + i: two such reads (k0 and k0 + 4) make one
// operand.
struct RhtB {
  u32x4 b[8][2];   // [kk][p]
};

typedef short rht_v4s __attribute__((ext_vector_type(4)));

__device__ __forceinline__ void rht_read_b(const RhtStage& st, RhtB& B) {
  const uint32_t lane = threadIdx.x & 63, g = lane >> 4, j = lane & 15, e = j >> 2, a = j & 3;
  const uint32_t hk = g >> 1, nb = g & 1, row = 8 * hk + e, f = rht_swz(e);
  const char* base = reinterpret_cast<const char*>(st.w);
  uint32_t off[2];
#pragma unroll
  for (int p = 0; p < 2; ++p) off[p] = row * 128 + 16 * ((4 * p + 2 * nb + (a >> 1)) ^ f) + 8 * (a & 1);
#pragma unroll
  for (int kk = 0; kk < 8; ++kk)
#pragma unroll
    for (int p = 0; p < 2; ++p)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const rht_v4s v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) rht_v4s*)(base + off[p] + kk * 2048 + h * 512));
        const uint2 w = __builtin_bit_cast(uint2, v);
        B.b[kk][p][2 * h] = w.x;
        B.b[kk][p][2 * h + 1] = w.y;
      }
}

// Half H of one tile from its raw words: acc[p][a'] is the 32x32 MFMA output block
// a = 2H + a' (output tokens 32a..32a+31) for column parity p of this lane's column
// pair.  Working in halves keeps 64 accumulators live instead of 128, which lets two
// waves share a SIMD.
template <int H>
__device__ __forceinline__ void rht_mma_half(const RhtRaw& raw, const u32x4 frag[8], f32x16 acc[2][2]) {
#pragma unroll
  for (int p = 0; p < 2; ++p)
#pragma unroll
    for (int a = 0; a < 2; ++a) acc[p][a] = f32x16{};
#pragma unroll
  for (int kk = 0; kk < 8; ++kk) {
    u32x4 b0, b1;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      b0[q] = __builtin_amdgcn_perm(raw.v[kk][2 * q + 1], raw.v[kk][2 * q], 0x05040100u);
      b1[q] = __builtin_amdgcn_perm(raw.v[kk][2 * q + 1], raw.v[kk][2 * q], 0x07060302u);
    }
    const bf16x8 v0 = __builtin_bit_cast(bf16x8, b0), v1 = __builtin_bit_cast(bf16x8, b1);
#pragma unroll
    for (int ap = 0; ap < 2; ++ap) {
      const int a = 2 * H + ap;
      const bf16x8 fa = a_operand(frag, a, kk);
      acc[0][ap] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa, v0, acc[0][ap], 0, 0, 0);
      acc[1][ap] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa, v1, acc[1][ap], 0, 0, 0);
    }
  }
}

// The same contraction from ready B operands (column slot n of pass p is tile column
// 32p + n); per output element the MFMA sums are the same as above.
template <int H>
__device__ __forceinline__ void rht_mma_half_b(const RhtB& B, const u32x4 frag[8], f32x16 acc[2][2]) {
#pragma unroll
  for (int p = 0; p < 2; ++p)
#pragma unroll
    for (int a = 0; a < 2; ++a) acc[p][a] = f32x16{};
#pragma unroll
  for (int kk = 0; kk < 8; ++kk) {
    const bf16x8 v0 = __builtin_bit_cast(bf16x8, B.b[kk][0]), v1 = __builtin_bit_cast(bf16x8, B.b[kk][1]);
#pragma unroll
    for (int ap = 0; ap < 2; ++ap) {
      const int a = 2 * H + ap;
      const bf16x8 fa = a_operand(frag, a, kk);
      acc[0][ap] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa, v0, acc[0][ap], 0, 0, 0);
      acc[1][ap] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa, v1, acc[1][ap], 0, 0, 0);
    }
  }
}

// Output token (within the chunk) of accumulator register r of block a for this lane.
__device__ __forceinline__ int acc_row(int a, int r) {
  const int hk = (threadIdx.x & 63) >> 5;
  return 32 * a + 8 * (r >> 2) + 4 * hk + (r & 3);
}

struct TileIter {
  int64_t ntiles, nslab, nchunk;
  __device__ TileIter(int64_t rows, int64_t cols) {
    nslab = (cols + 63) / 64;
    nchunk = rows / 128;
    ntiles = nslab * nchunk;
  }
  // tiles run slab-fastest: the waves in flight read whole token rows (every 64-column
  // slab of the same chunks), which keeps DRAM pages open; the column-wise output
  // lines they share (two chunks per 128-byte line) are completed within that window
  __device__ void decode(int64_t tile, int64_t& chunk, int64_t& slab) const {
    chunk = tile / nslab;
    slab = tile - chunk * nslab;
  }
};

// The wave's index in the grid, uniform (a scalar register) so that the tile
// arithmetic below stays off the vector ALUs.
__device__ __forceinline__ int64_t wave_id() {
  return (int64_t)blockIdx.x * (blockDim.x >> 6) + __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
}
__device__ __forceinline__ int64_t wave_count() { return ((int64_t)gridDim.x * blockDim.x) >> 6; }

// A wave's tiles wave_id(), wave_id() + step, ... with (chunk, slab) advanced by a
// fixed stride and one carry, so the loop divides only once.
struct TileWalk {
  int64_t nslab, ntiles, step, step_chunk, step_slab;
  int64_t tile, chunk, slab;
  __device__ TileWalk(int64_t rows, int64_t cols) {
    nslab = (cols + 63) / 64;
    ntiles = nslab * (rows / 128);
    step = wave_count();
    step_chunk = step / nslab;
    step_slab = step - step_chunk * nslab;
    tile = wave_id();
    chunk = tile / nslab;
    slab = tile - chunk * nslab;
  }
  __device__ bool valid() const { return tile < ntiles; }
  __device__ void next() {
    tile += step;
    chunk += step_chunk;
    slab += step_slab;
    if (slab >= nslab) {
      slab -= nslab;
      ++chunk;
    }
  }
};

// ---------------------------------------------------------------------------
// Standalone transform (bf16 in, f32 out); inverse uses H without input signs
// and applies s_t to the output rows.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_rht_bf16(const uint16_t* __restrict__ x, int64_t rows, int64_t cols,
                                                  RhtSigns sg, int inverse, float* __restrict__ y) {
  u32x4 frag[8];
  make_fragments(sg, !inverse, frag);
  const TileIter it(rows, cols);
  const int lane = threadIdx.x & 63;
  for (int64_t tile = wave_id(); tile < it.ntiles; tile += wave_count()) {
    int64_t chunk, slab;
    it.decode(tile, chunk, slab);
    const int64_t tok0 = chunk * 128, colp = slab * 64 + 2 * (lane & 31);
    const bool valid = colp < cols;
    RhtRaw raw;
    rht_load(x, cols, tok0, colp, valid, raw);
    auto emit = [&](const f32x16 (&acc)[2][2], int a0) {
#pragma unroll
      for (int ap = 0; ap < 2; ++ap)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int t = acc_row(a0 + ap, r);
          float v0 = acc[0][ap][r] * kRhtScale, v1 = acc[1][ap][r] * kRhtScale;
          if (inverse && ((sg.w[t >> 5] >> (t & 31)) & 1u)) { v0 = -v0; v1 = -v1; }
          if (valid) *reinterpret_cast<float2*>(y + (tok0 + t) * cols + colp) = make_float2(v0, v1);
        }
    };
    f32x16 acc[2][2];
    rht_mma_half<0>(raw, frag, acc);
    emit(acc, 0);
    rht_mma_half<1>(raw, frag, acc);
    emit(acc, 2);
  }
}

// ---------------------------------------------------------------------------
// Pass 1 of the fused path: amax of the transformed tensor.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void k_rht_amax(const uint16_t* __restrict__ x, int64_t rows, int64_t cols,
                                                  RhtSigns sg, AmaxSink sink) {
  __shared__ RhtStage stage[4];
  RhtStage& st = stage[__builtin_amdgcn_readfirstlane(threadIdx.x >> 6)];
  u32x4 frag[8];
  make_fragments(sg, true, frag);
  const int lane = threadIdx.x & 63;
  float m = 0.0f;
  TileWalk w(rows, cols);
  if (w.valid()) rht_issue<false>(x, cols, w.chunk * 128, w.slab * 64, st);
  for (; w.valid(); w.next()) {
    const int64_t col = w.slab * 64 + (lane & 31);   // column of pass 0; pass 1 is col + 32
    RhtB B;
    rht_wait_loads();
    rht_read_b(st, B);
    rht_wait_lds();
    TileWalk nw = w;
    nw.next();
    if (nw.valid()) rht_issue<false>(x, cols, nw.chunk * 128, nw.slab * 64, st);
    float t[2] = {0.0f, 0.0f};
    auto fold = [&](const f32x16 (&acc)[2][2]) {
#pragma unroll
      for (int p = 0; p < 2; ++p)
#pragma unroll
        for (int a = 0; a < 2; ++a)
#pragma unroll
          for (int r = 0; r < 16; ++r) t[p] = __builtin_fmaxf(t[p], __builtin_fabsf(acc[p][a][r]));
    };
    f32x16 acc[2][2];
    rht_mma_half_b<0>(B, frag, acc);
    fold(acc);
    rht_mma_half_b<1>(B, frag, acc);
    fold(acc);
    if (col < cols) m = __builtin_fmaxf(m, t[0]);
    if (col + 32 < cols) m = __builtin_fmaxf(m, t[1]);
  }
  // max |fl(acc*k)| = fl(max|acc| * k): scaling is monotone.  One atomic per
  // workgroup: same-address atomics serialize, so per-wave atomics would cost more
  // than the transform.
  __shared__ float wm[4];
  m = wave_max(m);
  if (lane == 0) wm[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0)
    post_amax(sink, __builtin_fmaxf(__builtin_fmaxf(wm[0], wm[1]), __builtin_fmaxf(wm[2], wm[3])) * kRhtScale);
}

// ---------------------------------------------------------------------------
// Pass 2: column-wise NVFP4 (blocks of 16 tokens) of the transformed tensor.
// After the permlane32 swaps each lane holds 16 consecutive tokens of one column.
// ---------------------------------------------------------------------------
// One operand of a column-wise pass: its tensor, shape, outputs, tensor scale and SR key.
struct RhtColOp {
  const uint16_t* x;
  int64_t rows, cols;
  uint8_t* ccodes;
  uint8_t* cscales;
  float gs;
  uint32_t k0, k1;
};

// Where a lane's outputs of one tile go.  Lane (n, hk) quantizes columns 64*slab + n
// (pass 0) and + 32 (pass 1).  Output block a of a column is 16 code bytes at 16 a of
// the column's 64-byte span in the tile, lane hk encoding bytes 8 hk..8 hk + 7; after
// blocks a and a + 1 the lane pair trades one half each, so lane 0 stores block a and
// lane 1 block a + 1 as whole 16-byte pieces.
// Addresses and counters are a wave-uniform part (scalar registers) plus one 32-bit
// lane part shared by both passes, which keeps the quantizer's vector registers free.
struct RhtTileOut {
  uint8_t* code_u[2];      // column 64 slab + 32 p, first token of the chunk
  uint8_t* scale_u[2];
  uint64_t idx8_u[2];      // SR: Philox counter of that column's first 8 tokens of the chunk
  uint32_t code_l, scale_l, idx8_l;   // lane (n, hk): column n's offset (scales, SR: plus its half)
  bool valid[2];
  uint32_t scale_word[2];
  uint2 prev[2];           // this lane's 8 code bytes of the last even block, pass p
};

// Codes of block a (8 bytes of this lane, pass p).  PAIR: held for an even a, stored
// with the held half for an odd a; otherwise stored as they are (the SR pass, whose
// registers are all taken by the draws, keeps the 8-byte stores).
template <bool PAIR>
__device__ __forceinline__ void rht_put_codes(RhtTileOut& t, int a, int p, uint2 w) {
  const uint32_t hk = (threadIdx.x & 63) >> 5;
  if constexpr (!PAIR) {
    if (t.valid[p]) *reinterpret_cast<uint2*>(t.code_u[p] + t.code_l + 8 * hk + 16 * a) = w;
    return;
  }
  if ((a & 1) == 0) {
    t.prev[p] = w;
    return;
  }
  // lanes >= 32 take lane hk = 0's half of block a; lanes < 32 hk = 1's half of block a - 1
  auto sx = __builtin_amdgcn_permlane32_swap(t.prev[p].x, w.x, false, false);
  auto sy = __builtin_amdgcn_permlane32_swap(t.prev[p].y, w.y, false, false);
  if (t.valid[p])
    *reinterpret_cast<uint4*>(t.code_u[p] + t.code_l + 16 * hk + 16 * (a - 1)) = make_uint4(sx[0], sy[0], sx[1],
                                                                                           sy[1]);
}

__device__ __forceinline__ RhtTileOut rht_tile_out(int64_t chunk, int64_t slab, const RhtColOp& o) {
  const uint32_t lane = threadIdx.x & 63, hk = lane >> 5, n = lane & 31;
  const int64_t half_rows = o.rows >> 1, nb = o.rows >> 4;
  const int64_t tok0 = chunk * 128;
  RhtTileOut t;
  // the lane parts stay below 2^32: 32 columns of a tensor with rows < 2^31
  t.code_l = n * (uint32_t)half_rows;
  t.scale_l = n * (uint32_t)nb + 4u * hk;
  t.idx8_l = n * (uint32_t)(o.rows >> 3) + 2u * hk;
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const int64_t c0 = slab * 64 + 32 * p;   // the column of lane n = 0
    t.valid[p] = c0 + n < o.cols;
    t.code_u[p] = o.ccodes + c0 * half_rows + (tok0 >> 1);
    t.scale_u[p] = o.cscales + c0 * nb + (tok0 >> 4);
    t.idx8_u[p] = (uint64_t)(c0 * o.rows + tok0) >> 3;
    t.scale_word[p] = 0u;
  }
  return t;
}

// Quantizes output block a of both passes from its accumulators.
template <bool SR>
__device__ __forceinline__ void rht_quant_block(const f32x16 (&acc)[2], int a, const RhtColOp& o,
                                                const RecipTable& rtab, RhtTileOut& t) {
  const float gs = o.gs;
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    if constexpr (!SR) {
      // RTN: the lane keeps its 8 values of each of the two 16-token blocks of output
      // block a (tokens 32a + 0..15: A, 16..31: B; registers 0..7 and 8..15) and trades
      // three words with the lane 32 away instead of regrouping the values: the partial
      // maxima, the scale codes and the packed codes.  Lane hk then owns block hk's outputs.
      float v[16];
      float mA = 0.0f, mB = 0.0f;
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        v[k] = (acc[p][k] * kRhtScale) * gs;
        if (k < 8) mA = __builtin_fmaxf(mA, __builtin_fabsf(v[k]));
        else mB = __builtin_fmaxf(mB, __builtin_fabsf(v[k]));
      }
      // lane hk = 0 receives the partner's A maximum, lane hk = 1 the partner's B one
      auto mx = __builtin_amdgcn_permlane32_swap(__float_as_uint(mA), __float_as_uint(mB), false, false);
      const float m = __builtin_fmaxf(__uint_as_float(mx[0]), __uint_as_float(mx[1]));
      const uint32_t sc = nvfp4_scale_code(m);   // scale of block hk
      auto scs = __builtin_amdgcn_permlane32_swap(sc, sc, false, false);   // every lane: (code A, code B)
      const RecipPair rpA = rtab.r[scs[0]], rpB = rtab.r[scs[1]];
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        v[k] = div2(v[k], rpA);
        v[8 + k] = div2(v[8 + k], rpB);
      }
      // nibbles of A: tokens 4hk + 0..3 then 8 + 4hk + 0..3; likewise for B
      const uint32_t wA = pack8_rtn(v, 1.0f), wB = pack8_rtn(v + 8, 1.0f);
      // lane hk = 0 now holds A's words of both halves, lane hk = 1 B's: the own
      // block's tokens 0..3 / 8..11 in the first word, 4..7 / 12..15 in the second
      auto wx = __builtin_amdgcn_permlane32_swap(wA, wB, false, false);
      const uint32_t lo = __builtin_amdgcn_perm(wx[1], wx[0], 0x05040100u);   // tokens 0..7
      const uint32_t hi = __builtin_amdgcn_perm(wx[1], wx[0], 0x07060302u);   // tokens 8..15
      rht_put_codes<true>(t, a, p, make_uint2(lo, hi));
      t.scale_word[p] |= sc << (8 * a);
    } else {
      // SR: regroup so that each lane holds 16 consecutive tokens of one block (lanes < 32
      // rows 0..15 of block a, lanes >= 32 rows 16..31), whose draws come from two
      // Philox evaluations.
      float v[16];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        auto s02 = __builtin_amdgcn_permlane32_swap(__float_as_uint(acc[p][j]), __float_as_uint(acc[p][8 + j]),
                                                    false, false);
        auto s13 = __builtin_amdgcn_permlane32_swap(__float_as_uint(acc[p][4 + j]),
                                                    __float_as_uint(acc[p][12 + j]), false, false);
        v[j] = __uint_as_float(s02[0]);
        v[4 + j] = __uint_as_float(s02[1]);
        v[8 + j] = __uint_as_float(s13[0]);
        v[12 + j] = __uint_as_float(s13[1]);
      }
      float m = 0.0f;
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        v[k] = (v[k] * kRhtScale) * gs;
        m = __builtin_fmaxf(m, __builtin_fabsf(v[k]));
      }
      const uint32_t sc = nvfp4_scale_code(m);
      const RecipPair rp = rtab.r[sc];
#pragma unroll
      for (int k = 0; k < 16; ++k) v[k] = div2(v[k], rp);
      uint32_t r0[8], r1[8];
      const uint64_t idx8 = t.idx8_u[p] + t.idx8_l + (uint64_t)(4 * a);   // 32 tokens per block a = 4 groups of 8
      sr_draws8(idx8, 1u, o.k0, o.k1, r0);
      sr_draws8(idx8 + 1, 1u, o.k0, o.k1, r1);
      const uint32_t w0 = pack8_sr(v, r0, 1.0f), w1 = pack8_sr(v + 8, r1, 1.0f);
      rht_put_codes<false>(t, a, p, make_uint2(w0, w1));
      t.scale_word[p] |= sc << (8 * a);
    }
  }
}

__device__ __forceinline__ void rht_store_scales(const RhtTileOut& t) {
  const int hk = (threadIdx.x & 63) >> 5;
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    // lane < 32 holds blocks 0,2,4,6 of the chunk and lane >= 32 blocks 1,3,5,7;
    // interleave so each lane stores four consecutive scale bytes.
    auto sw = __builtin_amdgcn_permlane32_swap(t.scale_word[p], t.scale_word[p], false, false);
    const uint32_t lo = hk ? sw[0] : t.scale_word[p];   // blocks 0,2,4,6
    const uint32_t hi = hk ? t.scale_word[p] : sw[1];   // blocks 1,3,5,7
    // bytes of lo: b0 b2 b4 b6, of hi: b1 b3 b5 b7
    const uint32_t first = __builtin_amdgcn_perm(hi, lo, 0x05010400u);   // b0 b1 b2 b3
    const uint32_t second = __builtin_amdgcn_perm(hi, lo, 0x07030602u);  // b4 b5 b6 b7
    if (t.valid[p]) *reinterpret_cast<uint32_t*>(t.scale_u[p] + t.scale_l) = hk ? second : first;
  }
}

template <bool SR>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void k_rht_nvfp4_col(const uint16_t* __restrict__ x, int64_t rows, int64_t cols,
                                                       RhtSigns sg, AmaxSource amax,
                                                       float* __restrict__ tensor_scale, uint8_t* __restrict__ ccodes,
                                                       uint8_t* __restrict__ cscales, uint32_t k0, uint32_t k1) {
  __shared__ RhtStage stage[4];
  __shared__ RecipTable rtab;
  RhtStage& st = stage[__builtin_amdgcn_readfirstlane(threadIdx.x >> 6)];
  fill_recip_table(rtab);
  __syncthreads();
  const RhtColOp op{x, rows, cols, ccodes, cscales, tensor_scale_publish(amax, tensor_scale), k0, k1};
  u32x4 frag[8];
  make_fragments(sg, true, frag);
  TileWalk w(rows, cols);
  if (!w.valid()) return;
  // Per tile: wait for its loads, read its B operands, start the next tile's loads into
  // the same buffer, then two halves of MFMAs (output blocks 2H, 2H + 1 of both column
  // passes), each followed by the quantization of its two blocks.  The quantization
  // waits for its half's MFMAs; the wave's SIMD partner keeps the vector ALUs busy
  // meanwhile (the two waves' VALU and MFMA work overlap).
  RhtB B;
  rht_issue<true>(x, cols, w.chunk * 128, w.slab * 64, st);
  for (; w.valid(); w.next()) {
    rht_wait_loads();
    rht_read_b(st, B);
    rht_wait_lds();
    {
      TileWalk nw = w;
      nw.next();
      if (nw.valid()) rht_issue<true>(x, cols, nw.chunk * 128, nw.slab * 64, st);
    }
    RhtTileOut t = rht_tile_out(w.chunk, w.slab, op);
    f32x16 acc[2][2];
    rht_mma_half_b<0>(B, frag, acc);
    {
      const f32x16 b0[2] = {acc[0][0], acc[1][0]};
      rht_quant_block<SR>(b0, 0, op, rtab, t);
      const f32x16 b1[2] = {acc[0][1], acc[1][1]};
      rht_quant_block<SR>(b1, 1, op, rtab, t);
    }
    rht_mma_half_b<1>(B, frag, acc);
    {
      const f32x16 b2[2] = {acc[0][0], acc[1][0]};
      rht_quant_block<SR>(b2, 2, op, rtab, t);
      const f32x16 b3[2] = {acc[0][1], acc[1][1]};
      rht_quant_block<SR>(b3, 3, op, rtab, t);
    }
    rht_store_scales(t);
  }
}

// ---------------------------------------------------------------------------
// fp32 input: VALU fast Walsh-Hadamard transform, one lane per (chunk, column) with the
// column's 128 tokens in registers (7 butterfly stages, 896 adds).  Sylvester H is the
// 7-fold Kronecker power of [[1, 1], [1, -1]], so stage h (h = 1, 2, ..., 64) pairs
// tokens i and i + h (i & h == 0) into (a + b, a - b); after the last stage v[i] is
// sum_t H[i][t] u[t].  Consecutive lanes take consecutive columns, so every token
// row is one coalesced 256-byte wave load.  The standalone transform, the amax pass
// and the column-wise quantizer call the same code, so all three see bitwise
// identical y = fl(v * fl(1/sqrt(128))).  fp32 operands would lose their low 16 bits
// on the bf16 MFMA path, and fp32 MFMA would run the dense contraction at 1/16 of the
// bf16 rate, while the transform itself is only 7 adds per element.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void fwht128(float (&v)[128]) {
#pragma unroll
  for (int h = 1; h < 128; h <<= 1)
#pragma unroll
    for (int i = 0; i < 128; ++i)
      if ((i & h) == 0) {
        const float a = v[i], b = v[i + h];
        v[i] = a + b;
        v[i + h] = a - b;
      }
}

// u[t] = s_t x[128 c + t][j] (forward) or x (inverse) for the column at `base`.
__device__ __forceinline__ void load_col128(const float* __restrict__ x, int64_t base, int64_t cols,
                                            const RhtSigns& sg, bool with_signs, float (&v)[128]) {
#pragma unroll
  for (int t = 0; t < 128; ++t) {
    const float a = x[base + (int64_t)t * cols];
    v[t] = (with_signs && ((sg.w[t >> 5] >> (t & 31)) & 1u)) ? -a : a;
  }
}

__global__ __launch_bounds__(256) void k_rht_f32(const float* __restrict__ x, int64_t rows, int64_t cols, RhtSigns sg,
                                                 int inverse, float* __restrict__ y) {
  const int64_t nchunk = rows / 128;
  const int64_t id = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (id >= nchunk * cols) return;
  const int64_t chunk = id / cols, j = id - chunk * cols;
  const int64_t base = chunk * 128 * cols + j;
  float v[128];
  load_col128(x, base, cols, sg, !inverse, v);
  fwht128(v);
#pragma unroll
  for (int t = 0; t < 128; ++t) {
    float o = v[t] * kRhtScale;
    if (inverse && ((sg.w[t >> 5] >> (t & 31)) & 1u)) o = -o;
    y[base + (int64_t)t * cols] = o;
  }
}

// Pass 1 for fp32: amax of the forward transform, max |fl(v k)| = fl(max |v| * k).
__global__ __launch_bounds__(256) void k_rht_amax_f32(const float* __restrict__ x, int64_t rows, int64_t cols,
                                                      RhtSigns sg, AmaxSink sink) {
  const int64_t nchunk = rows / 128;
  const int64_t id = (int64_t)blockIdx.x * 256 + threadIdx.x;
  float m = 0.0f;
  if (id < nchunk * cols) {
    const int64_t chunk = id / cols, j = id - chunk * cols;
    float v[128];
    load_col128(x, chunk * 128 * cols + j, cols, sg, true, v);
    fwht128(v);
#pragma unroll
    for (int t = 0; t < 128; ++t) m = __builtin_fmaxf(m, __builtin_fabsf(v[t]));
  }
  __shared__ float wm[4];
  m = wave_max(m);
  if ((threadIdx.x & 63) == 0) wm[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0)
    post_amax(sink, __builtin_fmaxf(__builtin_fmaxf(wm[0], wm[1]), __builtin_fmaxf(wm[2], wm[3])) * kRhtScale);
}

// Pass 2 for fp32: the lane holds the eight 16-token blocks of its column whole, so each
// block's maximum, scale and codes stay in the lane; its 64 code bytes and 8 scale bytes
// are contiguous in the column-wise layout and go out as four 16-byte and one 8-byte store.
template <bool SR>
__global__ __launch_bounds__(256) void k_rht_nvfp4_col_f32(const float* __restrict__ x, int64_t rows, int64_t cols,
                                                           RhtSigns sg, AmaxSource amax,
                                                           float* __restrict__ tensor_scale,
                                                           uint8_t* __restrict__ ccodes,
                                                           uint8_t* __restrict__ cscales, uint32_t k0, uint32_t k1) {
  __shared__ RecipTable rtab;
  fill_recip_table(rtab);
  __syncthreads();
  const float gs = tensor_scale_publish(amax, tensor_scale);
  const int64_t nchunk = rows / 128;
  const int64_t id = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (id >= nchunk * cols) return;
  const int64_t chunk = id / cols, j = id - chunk * cols;
  float v[128];
  load_col128(x, chunk * 128 * cols + j, cols, sg, true, v);
  fwht128(v);
  uint32_t w[16];
  uint32_t sc_lo = 0u, sc_hi = 0u;
#pragma unroll
  for (int b = 0; b < 8; ++b) {
    float* q = v + 16 * b;
    float m = 0.0f;
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      q[k] = (q[k] * kRhtScale) * gs;
      m = __builtin_fmaxf(m, __builtin_fabsf(q[k]));
    }
    const uint32_t sc = nvfp4_scale_code(m);
    const RecipPair rp = rtab.r[sc];
#pragma unroll
    for (int k = 0; k < 16; ++k) q[k] = div2(q[k], rp);
    if constexpr (SR) {
      uint32_t r0[8], r1[8];
      const uint64_t idx8 = (uint64_t)(j * rows + chunk * 128 + 16 * b) >> 3;
      sr_draws8(idx8, 1u, k0, k1, r0);
      sr_draws8(idx8 + 1, 1u, k0, k1, r1);
      w[2 * b] = pack8_sr(q, r0, 1.0f);
      w[2 * b + 1] = pack8_sr(q + 8, r1, 1.0f);
    } else {
      w[2 * b] = pack8_rtn(q, 1.0f);
      w[2 * b + 1] = pack8_rtn(q + 8, 1.0f);
    }
    if (b < 4) sc_lo |= sc << (8 * b);
    else sc_hi |= sc << (8 * (b - 4));
  }
  uint4* cd = reinterpret_cast<uint4*>(ccodes + j * (rows >> 1) + chunk * 64);
#pragma unroll
  for (int i = 0; i < 4; ++i) cd[i] = make_uint4(w[4 * i], w[4 * i + 1], w[4 * i + 2], w[4 * i + 3]);
  *reinterpret_cast<uint2*>(cscales + j * (rows >> 4) + chunk * 8) = make_uint2(sc_lo, sc_hi);
}

__global__ void k_zero1_rht(float* p) { *p = 0.0f; }

static RhtSigns pack_signs(const uint32_t s[4]) {
  RhtSigns r;
  for (int i = 0; i < 4; ++i) r.w[i] = s[i];
  return r;
}

// Persistent grid of at most `per_simd` waves per SIMD (256 CUs x 4 SIMDs).
static int rht_grid(int64_t rows, int64_t cols, int per_simd) {
  const int64_t tiles = ((cols + 63) / 64) * (rows / 128);
  const int64_t cap = (int64_t)1024 * per_simd;
  const int64_t waves = tiles < cap ? tiles : cap;
  return (int)((waves + 3) / 4);
}

// One lane per (128-row chunk, column).
static int lane_grid(int64_t rows, int64_t cols) { return (int)((rows / 128 * cols + 255) / 256); }

void launch_rht(const void* x, int dtype, int64_t rows, int64_t cols, const uint32_t signs[4], int inverse, float* y,
                hipStream_t st) {
  const RhtSigns sg = pack_signs(signs);
  if (dtype == 1) {
    k_rht_bf16<<<rht_grid(rows, cols, 1), 256, 0, st>>>(static_cast<const uint16_t*>(x), rows, cols, sg, inverse, y);
  } else {
    k_rht_f32<<<lane_grid(rows, cols), 256, 0, st>>>(static_cast<const float*>(x), rows, cols, sg, inverse, y);
  }
}

void launch_rht_amax(const void* x, bool f32, int64_t rows, int64_t cols, const uint32_t signs[4],
                     const AmaxSink& sink, hipStream_t st) {
  if (!sink.tp) k_zero1_rht<<<1, 1, 0, st>>>(sink.f);
  if (f32)
    k_rht_amax_f32<<<lane_grid(rows, cols), 256, 0, st>>>(static_cast<const float*>(x), rows, cols,
                                                          pack_signs(signs), sink);
  else
    k_rht_amax<<<rht_grid(rows, cols, 2), 256, 0, st>>>(static_cast<const uint16_t*>(x), rows, cols,
                                                       pack_signs(signs), sink);
}

void launch_rht_nvfp4_col(const void* xv, bool f32, int64_t rows, int64_t cols, const uint32_t signs[4], bool sr,
                          uint64_t seed, const AmaxSource& amax, float* tensor_scale, uint8_t* col_codes,
                          uint8_t* col_scales, hipStream_t st) {
  const uint32_t k0 = (uint32_t)seed, k1 = (uint32_t)(seed >> 32);
  const RhtSigns sg = pack_signs(signs);
  if (f32) {
    const float* xf = static_cast<const float*>(xv);
    if (sr)
      k_rht_nvfp4_col_f32<true><<<lane_grid(rows, cols), 256, 0, st>>>(xf, rows, cols, sg, amax, tensor_scale,
                                                                       col_codes, col_scales, k0, k1);
    else
      k_rht_nvfp4_col_f32<false><<<lane_grid(rows, cols), 256, 0, st>>>(xf, rows, cols, sg, amax, tensor_scale,
                                                                        col_codes, col_scales, k0, k1);
    return;
  }
  const uint16_t* x = static_cast<const uint16_t*>(xv);
  auto kern = sr ? k_rht_nvfp4_col<true> : k_rht_nvfp4_col<false>;
  kern<<<rht_grid(rows, cols, 2), 256, 0, st>>>(x, rows, cols, sg, amax, tensor_scale, col_codes, col_scales, k0, k1);
}

}  // namespace fp4q
