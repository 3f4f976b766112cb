// MXFP8 quantization for the attention Q/K projections (the 2D-block FP4
// training page keeps Q and K in MXFP8): E4M3 elements in 1x32 blocks, one
// UE8M0 scale per block, no tensor scale.  The scale is 2^e with e the
// smallest integer such that 448 * 2^e >= amax_B -- rounded up, as NVFP4
// paper App. B.4 does for MX scales so that no element saturates (the page
// ties saturation to MXFP8 convergence problems); element code = sign bit 7
// | E4M3 RNE code of |x * 2^-e|, four at a time through gfx950's packed
// FP8 convert (e4m3_pack4); one byte per element.
//
//   k_quant_mx8_row  ROWWISE: one thread per block of 32 consecutive bf16
//                    (four 16-byte loads, the next block's issued before the
//                    current one is encoded), 32 code bytes as two 16-byte
//                    stores
//   k_quant_mx8_col  COLWISE (codes of X^T): a 128 x 64 tile of X through
//                    LDS; a thread takes 16 rows of a column pair (half of
//                    a block of each column, the block amax completed with
//                    its neighbour lane), so the 8 lanes of a column write
//                    128 contiguous bytes of the X^T code row
//   k_dequant_mx8    codes x 2^e, fp32 or bf16
#include <hip/hip_runtime.h>

#include <stdint.h>

#include "fp4_device.hpp"
#include "fp4_internal.hpp"
#include "quant_common.hpp"

using namespace fp4dev;
using namespace fp4quant;

namespace {

constexpr int kBS = 32;
constexpr int kMx8Threads = 256;
constexpr int kMx8WgPerCu = 4;
constexpr int kColTileRows = 128;          // colwise tile: 128 rows (4 blocks) x 64 columns
constexpr int kColTileCols = 64;
// LDS words (bf16 pairs) of tile row r: r * 33 + (r / 16) * 8 -- rows one
// bank apart, and the 8 row groups of 16 that a column read touches at once
// start 24 banks apart, so the reads of a wave (8 column pairs x 8 groups)
// hit 64 distinct banks
__device__ __forceinline__ int col_tile_word(int r) { return r * 33 + (r >> 4) * 8; }
constexpr int kColTileWords = kColTileRows * 33 + 8 * 8;

// UE8M0 code and encode scale of a block: 2^e, e = min{e : 448 * 2^e >=
// amax} clamped to [-127, 127] (a zero block: e = -127).  With amax =
// m * 2^k, 1 <= m < 2: 448 = 1.75 * 2^8 covers it at e = k - 8 iff
// m <= 1.75, else at e = k - 7.
__device__ __forceinline__ uint32_t block_scale_mx8(float amax_b, float& s_enc_l) {
  int e = -127;
  if (amax_b > 0.0f) {
    const uint32_t b = __float_as_uint(amax_b);
    const int E = static_cast<int>(b >> 23);
    const uint32_t man = b & 0x7FFFFFu;
    int k;
    bool le;     // m <= 1.75
    if (E == 0) {  // fp32 subnormal: amax = man * 2^-149
      const int lead_pos = 31 - __clz(man);
      k = lead_pos - 149;
      const uint32_t lead = 1u << lead_pos;
      le = man <= lead + (lead >> 1) + (lead >> 2);
    } else {
      k = E - 127;
      le = man <= 0x600000u;
    }
    e = le ? k - 8 : k - 7;
    e = e < -127 ? -127 : (e > 127 ? 127 : e);
  }
  const int ne = -e;
  s_enc_l = ne >= -126 ? __uint_as_float(static_cast<uint32_t>(ne + 127) << 23)
                       : __uint_as_float(0x00400000u);
  return static_cast<uint32_t>(e + 127);
}

// Codes of a 32-element block, w[k] = elements 4k .. 4k + 3 in memory
// order; element code = sign bit 7 | E4M3 RNE magnitude of v * s.  The
// block scale 2^-e has 448 * 2^e >= amax, so |v * s| <= 448: the range in
// which the hardware convert of e4m3_pack4 is the format's RNE encoder.
// Counters: cnt[3] += |v * s| > 448 (kept for the counter contract; the
// bound makes it 0); cnt[4] += (v != 0 and magnitude code 0).
template <bool CNT>
__device__ __forceinline__ void encode_mx8(const float (&v)[kBS], float s, uint32_t (&w)[8],
                                           uint32_t (&cnt)[5]) {
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const float y[4] = {v[4 * k] * s, v[4 * k + 1] * s, v[4 * k + 2] * s, v[4 * k + 3] * s};
    w[k] = e4m3_pack4(y[0], y[1], y[2], y[3]);
    if constexpr (CNT) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        cnt[3] += fabsf(y[e]) > 448.0f ? 1u : 0u;
        cnt[4] += (v[4 * k + e] != 0.0f && ((w[k] >> (8 * e)) & 0x7Fu) == 0u) ? 1u : 0u;
      }
    }
  }
}

// The same for 16 elements (half a block), w[k] = elements 4k .. 4k + 3.
template <bool CNT>
__device__ __forceinline__ void encode_mx8_16(const float (&v)[16], float s, uint32_t (&w)[4],
                                              uint32_t (&cnt)[5]) {
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const float y[4] = {v[4 * k] * s, v[4 * k + 1] * s, v[4 * k + 2] * s, v[4 * k + 3] * s};
    w[k] = e4m3_pack4(y[0], y[1], y[2], y[3]);
    if constexpr (CNT) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        cnt[3] += fabsf(y[e]) > 448.0f ? 1u : 0u;
        cnt[4] += (v[4 * k + e] != 0.0f && ((w[k] >> (8 * e)) & 0x7Fu) == 0u) ? 1u : 0u;
      }
    }
  }
}

// ROWWISE: a grid-stride loop over blocks; the next block's loads are
// issued before the current block is encoded (past the end they re-read
// the current block, so no branch guards them).
template <bool CNT>
__global__ __launch_bounds__(kMx8Threads) void k_quant_mx8_row(
    const uint16_t* __restrict__ x, int64_t rows, int64_t cols, int64_t ld,
    uint8_t* __restrict__ codes, uint8_t* __restrict__ scales, fp4_counters* __restrict__ counters,
    int tiled) {
  const uint64_t bpr = static_cast<uint64_t>(cols) / kBS;
  const uint64_t n = static_cast<uint64_t>(rows) * bpr;
  const uint64_t kg = (bpr + 7) >> 3;
  const uint64_t stride = static_cast<uint64_t>(gridDim.x) * kMx8Threads;
  uint64_t i = static_cast<uint64_t>(blockIdx.x) * kMx8Threads + threadIdx.x;
  uint64_t r = bpr ? i / bpr : 0, j = bpr ? i - r * bpr : 0;
  const uint64_t sr = bpr ? stride / bpr : 0, sj = bpr ? stride - sr * bpr : 0;
  uint32_t cnt[5] = {0, 0, 0, 0, 0};
  uint4 q[4];
  if (i < n) {
    const uint4* src = reinterpret_cast<const uint4*>(x + r * ld + j * kBS);
#pragma unroll
    for (int k = 0; k < 4; ++k) q[k] = src[k];
  }
  for (; i < n; i += stride) {
    const uint64_t r_cur = r, j_cur = j;
    r += sr;
    j += sj;
    if (j >= bpr) {
      j -= bpr;
      ++r;
    }
    const bool has_next = i + stride < n;
    const uint4* nsrc = reinterpret_cast<const uint4*>(x + (has_next ? r : r_cur) * ld +
                                                       (has_next ? j : j_cur) * kBS);
    uint4 nq[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) nq[k] = nsrc[k];

    float v[kBS];
#pragma unroll
    for (int k = 0; k < 4; ++k) unpack8(q[k], v + 8 * k);
    float amax_b = 0.0f;
#pragma unroll
    for (int k = 0; k < kBS; ++k) amax_b = fmaxf(amax_b, fabsf(v[k]));
    float s;
    const uint32_t sc = block_scale_mx8(amax_b, s);
    uint32_t w[8];
    encode_mx8<CNT>(v, s, w, cnt);
    uint4* dst = reinterpret_cast<uint4*>(codes + r_cur * static_cast<uint64_t>(cols) + j_cur * kBS);
    dst[0] = make_uint4(w[0], w[1], w[2], w[3]);
    dst[1] = make_uint4(w[4], w[5], w[6], w[7]);
    scales[tiled ? tiled_scale_offset(r_cur, j_cur, kg) : r_cur * bpr + j_cur] =
        static_cast<uint8_t>(sc);
#pragma unroll
    for (int k = 0; k < 4; ++k) q[k] = nq[k];
  }
  if constexpr (CNT) flush_counters<kMx8Threads>(cnt, counters);
}

// COLWISE: tiles of 128 rows (4 blocks) x 64 columns of X.  Thread t =
// 8 p + h takes rows 16 h .. 16 h + 15 of columns 2p, 2p + 1 (one 32-bit
// LDS word per row holds both): half of block h / 2 of rows c0 + 2p and
// c0 + 2p + 1 of X^T; lanes t and t ^ 1 hold the two halves of a block and
// exchange their amaxes, and lanes 8p .. 8p + 7 write 128 contiguous code
// bytes of each of the two X^T rows.  Rows beyond X are whole blocks
// (rows % 32 == 0): both halves of a block are in or out together.
template <bool CNT>
__global__ __launch_bounds__(kMx8Threads) void k_quant_mx8_col(
    const uint16_t* __restrict__ x, int64_t rows, int64_t cols, int64_t ld,
    uint8_t* __restrict__ codes, uint8_t* __restrict__ scales, fp4_counters* __restrict__ counters,
    int tiled) {
  __shared__ uint32_t tile[kColTileWords];
  const int64_t tiles_r = (rows + kColTileRows - 1) / kColTileRows;
  const int64_t tiles_c = (cols + kColTileCols - 1) / kColTileCols;
  const uint64_t bpr_t = static_cast<uint64_t>(rows) / kBS;      // blocks per X^T row
  const uint64_t kg = (bpr_t + 7) >> 3;
  const int t = threadIdx.x;
  const int p = t >> 3, h = t & 7;
  uint32_t cnt[5] = {0, 0, 0, 0, 0};
  const int64_t n_tiles = tiles_r * tiles_c;
  // 128 rows x 64 columns = 1024 chunks of 8 bf16; chunk q = t + 256 k:
  // row q / 8, columns 8 (q % 8) ..; chunks outside X are neither loaded
  // nor staged.  The next tile's chunks are loaded into registers while the
  // current tile is encoded from LDS.
  uint4 u[4];
  auto load = [&](int64_t id) {
    const int64_t tr = id / tiles_c;
    const int64_t r0 = tr * kColTileRows, c0 = (id - tr * tiles_c) * kColTileCols;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int q = t + k * kMx8Threads;
      const int lr = q >> 3, lc = (q & 7) * 8;
      if (r0 + lr < rows && c0 + lc < cols)
        u[k] = *reinterpret_cast<const uint4*>(x + (r0 + lr) * ld + c0 + lc);
    }
  };
  if (blockIdx.x < n_tiles) load(blockIdx.x);
  for (int64_t tile_id = blockIdx.x; tile_id < n_tiles; tile_id += gridDim.x) {
    const int64_t tr = tile_id / tiles_c, tc = tile_id - tr * tiles_c;
    const int64_t r0 = tr * kColTileRows, c0 = tc * kColTileCols;
    __syncthreads();     // the previous tile's LDS reads are done
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int q = t + k * kMx8Threads;
      const int lr = q >> 3, lc = (q & 7) * 8;
      if (r0 + lr < rows && c0 + lc < cols) {
        uint32_t* d = tile + col_tile_word(lr) + (lc >> 1);
        d[0] = u[k].x;
        d[1] = u[k].y;
        d[2] = u[k].z;
        d[3] = u[k].w;
      }
    }
    __syncthreads();
    if (tile_id + gridDim.x < n_tiles) load(tile_id + gridDim.x);
    const int64_t row = r0 + 16 * h;          // first row of this thread's half block
    const bool rows_in = row < rows;          // the partner lane agrees (whole blocks)
    float v0[16], v1[16];
    float a0 = 0.0f, a1 = 0.0f;
    if (rows_in) {
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        const uint32_t w = tile[col_tile_word(16 * h + k) + p];
        v0[k] = bf16_to_f32(w & 0xFFFFu);
        v1[k] = bf16_to_f32(w >> 16);
        a0 = fmaxf(a0, fabsf(v0[k]));
        a1 = fmaxf(a1, fabsf(v1[k]));
      }
    }
    // the block amax: this half's and the neighbour lane's (max is exact)
    a0 = fmaxf(a0, __shfl_xor(a0, 1, 64));
    a1 = fmaxf(a1, __shfl_xor(a1, 1, 64));
    if (rows_in) {
      const uint64_t j = static_cast<uint64_t>(row) / kBS;
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int64_t c = c0 + 2 * p + e;
        if (c < cols) {
          float s;
          const uint32_t sc = block_scale_mx8(e ? a1 : a0, s);
          uint32_t w[4];
          encode_mx8_16<CNT>(e ? v1 : v0, s, w, cnt);
          *reinterpret_cast<uint4*>(codes + c * static_cast<uint64_t>(rows) + row) =
              make_uint4(w[0], w[1], w[2], w[3]);
          if ((h & 1) == 0)
            scales[tiled ? tiled_scale_offset(static_cast<uint64_t>(c), j, kg)
                         : static_cast<uint64_t>(c) * bpr_t + j] = static_cast<uint8_t>(sc);
        }
      }
    }
  }
  if constexpr (CNT) flush_counters<kMx8Threads>(cnt, counters);
}

// v = fp32(e4m3 * 2^e) (exact), fp32 or bf16 (RNE) out; one thread per block.
template <bool F32>
__global__ __launch_bounds__(kMx8Threads) void k_dequant_mx8(const uint8_t* __restrict__ codes,
                                                             const uint8_t* __restrict__ scales,
                                                             int64_t rows, int64_t cols,
                                                             void* __restrict__ out, int tiled) {
  const uint64_t bpr = static_cast<uint64_t>(cols) / kBS;
  const uint64_t n = static_cast<uint64_t>(rows) * bpr;
  const uint64_t kg = (bpr + 7) >> 3;
  for (uint64_t i = static_cast<uint64_t>(blockIdx.x) * kMx8Threads + threadIdx.x; i < n;
       i += static_cast<uint64_t>(gridDim.x) * kMx8Threads) {
    const uint64_t r = i / bpr, j = i - r * bpr;
    const float s = ue8m0_decode(scales[tiled ? tiled_scale_offset(r, j, kg) : i]);
    const uint4* src = reinterpret_cast<const uint4*>(codes + i * kBS);
    const uint4 a = src[0], b = src[1];
    const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
    float v[kBS];
#pragma unroll
    for (int k = 0; k < kBS; ++k) {
      const uint32_t c = (w[k >> 2] >> (8 * (k & 3))) & 0xFFu;
      const float m = scale_m3_decode<7>(c & 0x7Fu) * s;
      v[k] = (c & 0x80u) ? -m : m;
    }
    if constexpr (F32) {
      float4* dst = reinterpret_cast<float4*>(static_cast<float*>(out) + i * kBS);
#pragma unroll
      for (int k = 0; k < kBS / 4; ++k)
        dst[k] = make_float4(v[4 * k], v[4 * k + 1], v[4 * k + 2], v[4 * k + 3]);
    } else {
      uint32_t h[kBS / 2];
#pragma unroll
      for (int k = 0; k < kBS / 2; ++k) {
        uint32_t lo = __float_as_uint(v[2 * k]), hi = __float_as_uint(v[2 * k + 1]);
        lo = (lo + 0x7FFFu + ((lo >> 16) & 1u)) >> 16;
        hi = (hi + 0x7FFFu + ((hi >> 16) & 1u)) >> 16;
        h[k] = (lo & 0xFFFFu) | (hi << 16);
      }
      uint4* dst = reinterpret_cast<uint4*>(static_cast<uint16_t*>(out) + i * kBS);
#pragma unroll
      for (int k = 0; k < kBS / 8; ++k)
        dst[k] = make_uint4(h[4 * k], h[4 * k + 1], h[4 * k + 2], h[4 * k + 3]);
    }
  }
}

}  // namespace

namespace fp4lib {

hipError_t launch_quant_mx8(const QuantArgs& a, bool colwise, hipStream_t s) {
  if (a.rows > 0 && a.cols > 0) {
    if (colwise) {
      const int64_t tiles = ((a.rows + kColTileRows - 1) / kColTileRows) *
                            ((a.cols + kColTileCols - 1) / kColTileCols);
      const int64_t cap = grid_cap(kMx8WgPerCu);
      const int grid = static_cast<int>(tiles < cap ? tiles : cap);
      if (a.counters && a.count_elems)
        hipLaunchKernelGGL(k_quant_mx8_col<true>, dim3(grid), dim3(kMx8Threads), 0, s, a.x, a.rows,
                           a.cols, a.ld, a.codes, a.scales, a.counters, a.tiled);
      else
        hipLaunchKernelGGL(k_quant_mx8_col<false>, dim3(grid), dim3(kMx8Threads), 0, s, a.x,
                           a.rows, a.cols, a.ld, a.codes, a.scales, a.counters, a.tiled);
    } else {
      const uint64_t n = static_cast<uint64_t>(a.rows) * static_cast<uint64_t>(a.cols / kBS);
      const int grid = grid_for(n, kMx8WgPerCu, kMx8Threads);
      if (a.counters && a.count_elems)
        hipLaunchKernelGGL(k_quant_mx8_row<true>, dim3(grid), dim3(kMx8Threads), 0, s, a.x, a.rows,
                           a.cols, a.ld, a.codes, a.scales, a.counters, a.tiled);
      else
        hipLaunchKernelGGL(k_quant_mx8_row<false>, dim3(grid), dim3(kMx8Threads), 0, s, a.x,
                           a.rows, a.cols, a.ld, a.codes, a.scales, a.counters, a.tiled);
    }
  }
  return hipGetLastError();
}

hipError_t launch_dequant_mx8(int tiled, const uint8_t* codes, const uint8_t* scales, int64_t rows,
                              int64_t cols, void* out, int out_fp32, hipStream_t s) {
  if (rows > 0 && cols > 0) {
    const uint64_t n = static_cast<uint64_t>(rows) * static_cast<uint64_t>(cols / kBS);
    const int grid = grid_for(n, 2, kMx8Threads);
    if (out_fp32)
      hipLaunchKernelGGL(k_dequant_mx8<true>, dim3(grid), dim3(kMx8Threads), 0, s, codes, scales,
                         rows, cols, out, tiled);
    else
      hipLaunchKernelGGL(k_dequant_mx8<false>, dim3(grid), dim3(kMx8Threads), 0, s, codes, scales,
                         rows, cols, out, tiled);
  }
  return hipGetLastError();
}

}  // namespace fp4lib
