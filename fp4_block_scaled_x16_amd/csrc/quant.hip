// gfx950 kernels for the quantization side of FP4 block scaling:
//   tensor amax (plain and in the RHT-rotated space), rowwise 1D quantizer,
//   colwise (transposing) 1D quantizer with optional fused 16-point RHT,
//   the two together from one read of X (dual), 16x16 2D quantizer emitting
//   W and W^T codes, dequantizer, standalone RHT.
//
// All of these are HBM-bound streams: every kernel reads its bf16 input
// once with 16-byte vector loads, keeps the block in registers (and LDS
// where a transpose is needed), and writes codes/scales with the widest
// contiguous stores the layout allows.  Grids are capped at a few
// workgroups per CU and walk the work with grid-stride loops, so the
// tensor-scale prologue and the counter flush are paid once per workgroup.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <stdint.h>

#include "fp4_device.hpp"
#include "fp4_internal.hpp"
#include "quant_common.hpp"

using namespace fp4dev;
using namespace fp4quant;

namespace {

constexpr int kThreads = 256;       // tiled kernels (colwise, 2D)
constexpr int kStream = 512;        // streaming kernels (amax, rowwise, dequant, RHT)
// Resident workgroups per CU of the persistent quantizer grids (measured on
// MI355X: more waves let the VALU-heavy stochastic-rounding kernels overlap
// their LDS and memory latency; the RNE tile kernels prefer fewer).
constexpr int kRowWgPerCu = 2;      // rowwise, RNE and SR
constexpr int kColWgPerCuSR = 6;    // colwise and dual with stochastic rounding
constexpr int kTileWgPerCu = 3;     // colwise / dual RNE, 2D
constexpr int kAmaxWgPerCu = 1;     // tensor amax (plain and 16-point RHT)

// ---------------------------------------------------------------- amax --
__global__ void k_fill_u32(uint32_t* p, uint32_t v) { *p = v; }

// Workgroup max of a per-thread value (fp32 bits of a magnitude), then one
// atomic max -- skipped when the current value is already as large.
template <int NT>
__device__ __forceinline__ void flush_max(uint32_t m, uint32_t* out) {
  __shared__ uint32_t red[NT / 64];
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) m = max(m, static_cast<uint32_t>(__shfl_xor(m, o, 64)));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
#pragma unroll
    for (int w = 1; w < NT / 64; ++w) m = max(m, red[w]);
    if (m > __hip_atomic_load(out, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) atomicMax(out, m);
  }
}

// Two maxima at once (one barrier): a -> *out_a, and b -> *out_b if out_b.
template <int NT>
__device__ __forceinline__ void flush_max2(uint32_t a, uint32_t b, uint32_t* out_a,
                                           uint32_t* out_b) {
  __shared__ uint32_t red[NT / 64][2];
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    a = max(a, static_cast<uint32_t>(__shfl_xor(a, o, 64)));
    b = max(b, static_cast<uint32_t>(__shfl_xor(b, o, 64)));
  }
  if ((threadIdx.x & 63) == 0) {
    red[threadIdx.x >> 6][0] = a;
    red[threadIdx.x >> 6][1] = b;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
#pragma unroll
    for (int w = 1; w < NT / 64; ++w) {
      a = max(a, red[w][0]);
      b = max(b, red[w][1]);
    }
    if (a > __hip_atomic_load(out_a, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) atomicMax(out_a, a);
    if (out_b && b > __hip_atomic_load(out_b, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT))
      atomicMax(out_b, b);
  }
}

// max |x| over a [rows, cols] bf16 matrix, cols % 8 == 0.  |x| as fp32 bits
// is monotone in the value, so an unsigned atomic max is exact.
__global__ __launch_bounds__(kStream) void k_amax(const uint16_t* __restrict__ x, int64_t rows,
                                                  int64_t cols, int64_t ld,
                                                  uint32_t* __restrict__ out) {
  const uint64_t cpr = static_cast<uint64_t>(cols) >> 3;      // 16-byte chunks per row
  const uint64_t n = static_cast<uint64_t>(rows) * cpr;
  const uint64_t stride = static_cast<uint64_t>(gridDim.x) * kStream;
  uint64_t i = static_cast<uint64_t>(blockIdx.x) * kStream + threadIdx.x;
  uint64_t r = cpr ? i / cpr : 0, j = cpr ? i - r * cpr : 0;
  const uint64_t sr = cpr ? stride / cpr : 0, sj = cpr ? stride - sr * cpr : 0;
  // two 16-byte chunks per thread and iteration, loads issued together
  uint32_t m = 0;
  for (; i < n; i += 2 * stride) {
    const uint64_t r1 = r, j1 = j;
    r += sr;
    j += sj;
    if (j >= cpr) {
      j -= cpr;
      ++r;
    }
    const bool two = i + stride < n;
    const uint4 q0 = *reinterpret_cast<const uint4*>(x + r1 * ld + j1 * 8);
    const uint4 q1 = *reinterpret_cast<const uint4*>(x + (two ? r : r1) * ld + (two ? j : j1) * 8);
    r += sr;
    j += sj;
    if (j >= cpr) {
      j -= cpr;
      ++r;
    }
    // |bf16| as unsigned 16-bit halves; the max of magnitudes is monotone
    const uint32_t w[8] = {q0.x, q0.y, q0.z, q0.w, q1.x, q1.y, q1.z, q1.w};
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const uint32_t a = w[k] & 0x7FFF7FFFu;
      m = max(m, max(a & 0xFFFFu, a >> 16));
    }
  }
  m <<= 16;   // fp32 bits of the largest magnitude
  flush_max<kStream>(m, out);
}

// max |(1/4) D_r H16 v| over every 16-row group v of every column, and (if
// out_plain) max |x| over the same values before the rotation, from the
// same read.  One thread per (column pair, group); rows % 16 == 0,
// cols % 8 == 0.
__global__ __launch_bounds__(kStream) void k_amax_rht(const uint16_t* __restrict__ x,
                                                      int64_t rows, int64_t cols, int64_t ld,
                                                      uint32_t signs, uint32_t* __restrict__ out,
                                                      uint32_t* __restrict__ out_plain) {
  const uint64_t pairs = static_cast<uint64_t>(cols) >> 1;
  const uint64_t n = (static_cast<uint64_t>(rows) >> 4) * pairs;
  const uint64_t stride = static_cast<uint64_t>(gridDim.x) * kStream;
  float m = 0.0f;
  uint32_t mp = 0;   // largest |x| as bf16 magnitude bits, as k_amax takes it
  for (uint64_t i = static_cast<uint64_t>(blockIdx.x) * kStream + threadIdx.x; i < n;
       i += stride) {
    const uint64_t g = i / pairs, p = i - g * pairs;
    const uint16_t* src = x + g * 16 * ld + p * 2;
    float a[16], b[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const uint32_t w = *reinterpret_cast<const uint32_t*>(src + k * ld);
      a[k] = bf16_to_f32(w & 0xFFFFu);
      b[k] = bf16_to_f32(w >> 16);
      const uint32_t mag = w & 0x7FFF7FFFu;
      mp = max(mp, max(mag & 0xFFFFu, mag >> 16));
    }
    rht16(a, signs);
    rht16(b, signs);
#pragma unroll
    for (int k = 0; k < 16; ++k) m = fmaxf(m, fmaxf(fabsf(a[k]), fabsf(b[k])));
  }
  flush_max2<kStream>(__float_as_uint(m), mp << 16, out, out_plain);
}

// ------------------------------------------------------ rowwise 1D ------
// One thread per block of BS consecutive elements of a row.  With RHT
// (16-element blocks) every N-element group of a row is rotated first
// (NVFP4 paper §4.2: the Fprop / Dgrad operands, rotated along K): the
// grid stride is a multiple of 64, so lane l handles blocks i = l mod 64,
// and the N / 16 blocks of a group (cols % N == 0) sit on consecutive
// lanes with the same bits above N / 16, which rht_n combines by shuffles.
template <int FMT, int RND, int CNT, bool RHT = false>
__global__ __launch_bounds__(kStream) void k_quant_row(
    const uint16_t* __restrict__ x, int64_t rows, int64_t cols, int64_t ld,
    uint8_t* __restrict__ codes, uint8_t* __restrict__ scales, const float* __restrict__ amax,
    float target, float* __restrict__ s_dec_out, uint64_t seed, uint64_t offset,
    fp4_counters* __restrict__ counters, int tiled, int scale_up, RhtN rht) {
  constexpr int BS = FMT == kMX ? 32 : 16;
  float s_enc_g = 1.0f, s_dec_g = 1.0f;
  if constexpr (FMT != kMX) global_scales(*amax, target, s_enc_g, s_dec_g);
  if (s_dec_out && blockIdx.x == 0 && threadIdx.x == 0) *s_dec_out = s_dec_g;
  __shared__ float enc_tab[FMT == kMX ? 1 : 256];
  fill_enc_table<FMT, kStream>(enc_tab, s_dec_g);
  if constexpr (FMT != kMX) __syncthreads();

  const uint64_t bpr = static_cast<uint64_t>(cols) / BS;
  const uint64_t n = static_cast<uint64_t>(rows) * bpr;
  const uint64_t stride = static_cast<uint64_t>(gridDim.x) * kStream;
  uint64_t i = static_cast<uint64_t>(blockIdx.x) * kStream + threadIdx.x;
  uint64_t r = bpr ? i / bpr : 0, j = bpr ? i - r * bpr : 0;
  const uint64_t sr = bpr ? stride / bpr : 0, sj = bpr ? stride - sr * bpr : 0;
  uint32_t cnt[5] = {0, 0, 0, 0, 0};
  // The next block's loads are issued before the current block is encoded;
  // past the end they re-read a valid block, so no branch guards them.
  uint4 q[BS / 8];
  if (i < n) {
    const uint4* src = reinterpret_cast<const uint4*>(x + r * ld + j * BS);
#pragma unroll
    for (int k = 0; k < BS / 8; ++k) q[k] = src[k];
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
                                                       (has_next ? j : j_cur) * BS);
    uint4 nq[BS / 8];
#pragma unroll
    for (int k = 0; k < BS / 8; ++k) nq[k] = nsrc[k];

    float v[BS];
#pragma unroll
    for (int k = 0; k < BS / 8; ++k) unpack8(q[k], v + 8 * k);
    if constexpr (RHT && BS == 16) rht_n(v, rht, static_cast<int>(threadIdx.x & 7));
    float amax_b = 0.0f;
#pragma unroll
    for (int k = 0; k < BS; ++k) amax_b = fmaxf(amax_b, fabsf(v[k]));
    float s_enc_l;
    const uint32_t sc =
        scale_for_block<FMT>(amax_b, s_enc_g, s_dec_g, s_enc_l, cnt, scale_up, enc_tab);
    uint32_t words[BS / 8];
    encode_block<BS, RND, CNT == 2>(v, s_enc_l, r_cur * static_cast<uint64_t>(cols) + j_cur * BS, seed,
                               offset, words, cnt);
    uint8_t* dst = codes + r_cur * (static_cast<uint64_t>(cols) >> 1) + j_cur * (BS / 2);
    if constexpr (BS == 16) {
      *reinterpret_cast<uint2*>(dst) = make_uint2(words[0], words[1]);
    } else {
      *reinterpret_cast<uint4*>(dst) = make_uint4(words[0], words[1], words[2], words[3]);
    }
    scales[tiled ? tiled_scale_offset(r_cur, j_cur, (bpr + 7) >> 3) : r_cur * bpr + j_cur] =
        static_cast<uint8_t>(sc);
#pragma unroll
    for (int k = 0; k < BS / 8; ++k) q[k] = nq[k];
  }
  if constexpr (CNT) flush_counters<kStream>(cnt, counters);
}

// ------------------------------------------- transposing LDS tile ------
// The colwise and dual quantizers stage a tile of 8 BS rows x 64 bf16
// columns of X in LDS: each row is eight 16-byte chunks, written by row
// (one lane per chunk or block) and read by column (lane (grp, pair) reads
// 32-bit word `pair` of rows grp * BS + k).  Chunk c of row r sits at
//   r * 8 + (r / BS) * 8 + (c ^ f(r)),
// f(r) = (r / BS) & 7 ^ (low bits of r): the XOR puts the eight row groups a
// column read touches at once in eight different chunk columns, and the
// rows that one 16-byte write instruction covers (2 or 4 consecutive rows)
// in different chunk columns too; the one-chunk pad after each group of BS
// rows alternates the group's 128-byte bank half, so neither pattern
// conflicts with 32 or with 64 four-byte banks.
template <int BS>
__device__ __forceinline__ int tile_chunk(int r, int c) {
  const int f = ((r / BS) & 7) ^ (BS == 16 ? ((r ^ (r >> 1)) & 1) : ((r ^ (r >> 2)) & 3));
  return r * 8 + (r / BS) * 8 + (c ^ f);
}

template <int BS>
constexpr int kTileChunks = 8 * BS * 8 + 8 * 8;

// 32-bit word p (0..31: bf16 columns 2p, 2p + 1) of tile row r.
template <int BS>
__device__ __forceinline__ uint32_t tile_word(const uint4* tile, int r, int p) {
  return reinterpret_cast<const uint32_t*>(tile)[tile_chunk<BS>(r, p >> 2) * 4 + (p & 3)];
}

// ------------------------------------------------------ colwise 1D ------
// Quantizes X^T: blocks are BS consecutive rows of one column.  A workgroup
// stages a (8 BS) x 64 tile of X in LDS (coalesced 16-byte row loads), then
// each thread takes one column pair and one row group, optionally rotates
// each 16-row group by the RHT, and writes the codes of X^T so that the 8
// lanes of a column cover 8 consecutive groups (64 or 128 contiguous bytes).
//
// AMX (amax only): the same staging and rotation, but instead of encoding,
// the largest |value| is reduced into *amax_out (fp32 bits, atomic max):
// the tensor amax in the rotated space for the N-point RHT variants.
template <int FMT, int RND, bool RHT, int CNT, bool AMX = false>
__global__ __launch_bounds__(kThreads) void k_quant_col(
    const uint16_t* __restrict__ x, int64_t rows, int64_t cols, int64_t ld,
    uint8_t* __restrict__ codes, uint8_t* __restrict__ scales, const float* __restrict__ amax,
    float target, float* __restrict__ s_dec_out, uint64_t seed, uint64_t offset,
    RhtN rht, fp4_counters* __restrict__ counters, int tiled, uint32_t* __restrict__ amax_out,
    int scale_up) {
  constexpr int BS = FMT == kMX ? 32 : 16;
  constexpr int TR = 8 * BS;        // tile rows (8 groups)
  constexpr int TC = 64;            // tile columns
  __shared__ uint4 tile[kTileChunks<BS>];

  float s_enc_g = 1.0f, s_dec_g = 1.0f;
  if constexpr (FMT != kMX && !AMX) global_scales(*amax, target, s_enc_g, s_dec_g);
  if (s_dec_out && blockIdx.x == 0 && threadIdx.x == 0) *s_dec_out = s_dec_g;
  // read after the first tile's barrier
  __shared__ float enc_tab[FMT == kMX || AMX ? 1 : 256];
  if constexpr (!AMX) fill_enc_table<FMT, kThreads>(enc_tab, s_dec_g);

  // tile counts fit in 32 bits (the host keeps rows, cols below 2^31)
  const uint32_t tiles_c = static_cast<uint32_t>((cols + TC - 1) / TC);
  const uint32_t tiles_r = static_cast<uint32_t>((rows + TR - 1) / TR);
  const uint32_t ntiles = tiles_c * tiles_r;
  const int t = threadIdx.x;
  const int lane = t & 63, wave = t >> 6;
  const int grp = lane & 7;                  // row group handled in the compute phase
  const int pair = wave * 8 + (lane >> 3);   // column pair (0..31)
  uint32_t cnt[5] = {0, 0, 0, 0, 0};
  float vmax = 0.0f;                         // AMX

  for (uint32_t tile_id = blockIdx.x; tile_id < ntiles; tile_id += gridDim.x) {
    const uint32_t tr = tile_id / tiles_c, tc = tile_id - tr * tiles_c;
    const int64_t r0 = static_cast<int64_t>(tr) * TR, c0 = static_cast<int64_t>(tc) * TC;
    // load: TR rows x 8 chunks of 16 bytes
#pragma unroll
    for (int k = 0; k < TR * 8 / kThreads; ++k) {
      const int chunk = t + k * kThreads;
      const int lr = chunk >> 3, lc = (chunk & 7) * 8;
      uint4 q = make_uint4(0, 0, 0, 0);
      if (r0 + lr < rows && c0 + lc < cols)
        q = *reinterpret_cast<const uint4*>(x + (r0 + lr) * ld + c0 + lc);
      tile[tile_chunk<BS>(lr, chunk & 7)] = q;
    }
    __syncthreads();
    const int64_t col = c0 + 2 * pair;
    const int64_t row = r0 + grp * BS;
    if (col < cols && row < rows) {
      // the two columns one after the other: half the live registers
#pragma unroll 1
      for (int h = 0; h < 2; ++h) {
        float v[BS];
#pragma unroll
        for (int k = 0; k < BS; ++k) {
          const uint32_t w = tile_word<BS>(tile, grp * BS + k, pair);
          v[k] = bf16_to_f32(h ? (w >> 16) : (w & 0xFFFFu));
        }
        if constexpr (RHT) rht_n(*reinterpret_cast<float(*)[16]>(v), rht, grp);
        const int64_t c = col + h;
        float amax_b = 0.0f;
#pragma unroll
        for (int k = 0; k < BS; ++k) amax_b = fmaxf(amax_b, fabsf(v[k]));
        if constexpr (AMX) {
          vmax = fmaxf(vmax, amax_b);
          continue;
        }
        float s_enc_l;
        const uint32_t sc =
            scale_for_block<FMT>(amax_b, s_enc_g, s_dec_g, s_enc_l, cnt, scale_up, enc_tab);
        uint32_t words[BS / 8];
        encode_block<BS, RND, CNT == 2>(v, s_enc_l, static_cast<uint64_t>(c) * rows + row, seed,
                                   offset, words, cnt);
        uint8_t* dst = codes + c * (rows >> 1) + (row >> 1);
        if constexpr (BS == 16) {
          *reinterpret_cast<uint2*>(dst) = make_uint2(words[0], words[1]);
        } else {
          *reinterpret_cast<uint4*>(dst) = make_uint4(words[0], words[1], words[2], words[3]);
        }
        const uint64_t kb = static_cast<uint64_t>(rows / BS);
        scales[tiled ? tiled_scale_offset(c, row / BS, (kb + 7) >> 3) : c * kb + row / BS] =
            static_cast<uint8_t>(sc);
      }
    }
    __syncthreads();
  }
  if constexpr (AMX) flush_max<kThreads>(__float_as_uint(vmax), amax_out);
  if constexpr (CNT) flush_counters<kThreads>(cnt, counters);
}

// ------------------------------------------------ dual: rowwise + colwise --
// One read of X for both code matrices a linear layer takes from it: the
// rowwise codes (blocks along cols: the Fprop / Dgrad operand) and the codes
// of X^T (blocks along rows, optionally RHT-rotated: the Wgrad operand,
// NVFP4 paper §4.1 and §4.2).  A workgroup walks (8 BS) x 64 tiles of X as
// k_quant_col does.  Each thread loads two whole rowwise blocks of the tile
// (BS consecutive elements of a row each), encodes them from registers as
// k_quant_row does, and stores them into the LDS tile; the colwise half
// then runs from LDS exactly as k_quant_col.  The next tile's loads are
// issued before the current tile is encoded.  Both halves use the same
// rounding mode, each with its own tensor scale, Philox key and counter
// offset, and output layout.  RHT rotates the colwise side's N-row groups
// (any N); RRHT rotates the rowwise side's blocks along the row (N = 4 or
// 16, within a block: the Fprop / Dgrad operands, §4.2).
template <int FMT, int RND, bool RHT, int CNT, bool RRHT = false>
__global__ __launch_bounds__(kThreads)
__attribute__((amdgpu_waves_per_eu(FMT == kMX ? 1 : 3))) void k_quant_dual(
    const uint16_t* __restrict__ x, int64_t rows, int64_t cols, int64_t ld,
    uint8_t* __restrict__ codes, uint8_t* __restrict__ scales, uint8_t* __restrict__ codes_t,
    uint8_t* __restrict__ scales_t, const float* __restrict__ amax,
    const float* __restrict__ amax_t, float target, float target_t,
    float* __restrict__ s_dec_out, float* __restrict__ s_dec_t_out, uint64_t seed,
    uint64_t offset, uint64_t seed_t, uint64_t offset_t, RhtN rht,
    fp4_counters* __restrict__ counters, int tiled, int tiled_t, int scale_up, int scale_up_t,
    RhtN rht_row) {
  constexpr int BS = FMT == kMX ? 32 : 16;
  constexpr int TR = 8 * BS;        // tile rows (8 groups)
  constexpr int TC = 64;            // tile columns
  constexpr int BPR = TC / BS;      // rowwise blocks per tile row
  constexpr int NB = TR * BPR / kThreads;   // rowwise blocks per thread and tile (2)
  static_assert(NB * kThreads == TR * BPR, "tile must split evenly into blocks");
  __shared__ uint4 tile[kTileChunks<BS>];

  float s_enc_g = 1.0f, s_dec_g = 1.0f, s_enc_gt = 1.0f, s_dec_gt = 1.0f;
  if constexpr (FMT != kMX) {
    global_scales(*amax, target, s_enc_g, s_dec_g);
    global_scales(*amax_t, target_t, s_enc_gt, s_dec_gt);
  }
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    if (s_dec_out) *s_dec_out = s_dec_g;
    if (s_dec_t_out) *s_dec_t_out = s_dec_gt;
  }
  __shared__ float enc_tab[2][FMT == kMX ? 1 : 256];   // rowwise, colwise side
  fill_enc_table<FMT, kThreads>(enc_tab[0], s_dec_g);
  fill_enc_table<FMT, kThreads>(enc_tab[1], s_dec_gt);
  if constexpr (FMT != kMX) __syncthreads();

  // tile counts fit in 32 bits (the host keeps rows, cols below 2^31)
  const uint32_t tiles_c = static_cast<uint32_t>((cols + TC - 1) / TC);
  const uint32_t tiles_r = static_cast<uint32_t>((rows + TR - 1) / TR);
  const uint32_t ntiles = tiles_c * tiles_r;
  const uint64_t bpr = static_cast<uint64_t>(cols) / BS;   // rowwise blocks per row of X
  const int t = threadIdx.x;
  const int lane = t & 63, wave = t >> 6;
  const int grp = lane & 7;                  // row group handled in the colwise phase
  const int pair = wave * 8 + (lane >> 3);   // column pair (0..31)
  uint32_t cnt[5] = {0, 0, 0, 0, 0};

  // rowwise block b = t + k * kThreads of a tile: tile row b / BPR, columns
  // (b % BPR) * BS ..; blocks outside X load zeros and write nothing
  auto load = [&](uint32_t tile_id, uint4 (&q)[NB][BS / 8]) {
    const uint32_t tr = tile_id / tiles_c, tc = tile_id - tr * tiles_c;
#pragma unroll
    for (int k = 0; k < NB; ++k) {
      const int b = t + k * kThreads;
      const int64_t r = static_cast<int64_t>(tr) * TR + b / BPR;
      const int64_t c = static_cast<int64_t>(tc) * TC + (b % BPR) * BS;
      const bool in = tile_id < ntiles && r < rows && c < cols;
#pragma unroll
      for (int e = 0; e < BS / 8; ++e)
        q[k][e] = in ? *reinterpret_cast<const uint4*>(x + r * ld + c + 8 * e)
                     : make_uint4(0, 0, 0, 0);
    }
  };

  uint4 q[NB][BS / 8];
  load(blockIdx.x, q);
  for (uint32_t tile_id = blockIdx.x; tile_id < ntiles; tile_id += gridDim.x) {
    const uint32_t tr = tile_id / tiles_c, tc = tile_id - tr * tiles_c;
    const int64_t r0 = static_cast<int64_t>(tr) * TR, c0 = static_cast<int64_t>(tc) * TC;
    uint4 nq[NB][BS / 8];
    load(tile_id + gridDim.x, nq);
#pragma unroll
    for (int k = 0; k < NB; ++k) {
      const int b = t + k * kThreads;
      const int lr = b / BPR, lc = (b % BPR) * BS;
      const int64_t r = r0 + lr, c = c0 + lc;
#pragma unroll
      for (int e = 0; e < BS / 8; ++e) tile[tile_chunk<BS>(lr, lc / 8 + e)] = q[k][e];
      float v[BS];
#pragma unroll
      for (int e = 0; e < BS / 8; ++e) unpack8(q[k][e], v + 8 * e);
      if constexpr (RRHT && BS == 16) rht_n(v, rht_row, 0);   // N <= 16: no shuffles
      float amax_b = 0.0f;
#pragma unroll
      for (int e = 0; e < BS; ++e) amax_b = fmaxf(amax_b, fabsf(v[e]));
      float s_enc_l;
      const bool in = r < rows && c < cols;
      uint32_t sc_cnt[5] = {0, 0, 0, 0, 0};
      const uint32_t sc =
          scale_for_block<FMT>(amax_b, s_enc_g, s_dec_g, s_enc_l, sc_cnt, scale_up, enc_tab[0]);
      if (in) {
        cnt[0] += sc_cnt[0];
        cnt[1] += sc_cnt[1];
        cnt[2] += sc_cnt[2];
      }
      uint32_t words[BS / 8];
      // without the RHT both sides quantize the same values: the nonzero
      // inputs are counted here for both; a rotated side counts its own
      encode_block<BS, RND, CNT == 2, (RHT || RRHT) ? 1 : 2>(
          v, s_enc_l, static_cast<uint64_t>(r) * cols + c, seed, offset, words, cnt);
      if (in) {
        uint8_t* dst = codes + r * (cols >> 1) + (c >> 1);
        if constexpr (BS == 16) {
          *reinterpret_cast<uint2*>(dst) = make_uint2(words[0], words[1]);
        } else {
          *reinterpret_cast<uint4*>(dst) = make_uint4(words[0], words[1], words[2], words[3]);
        }
        const uint64_t j = static_cast<uint64_t>(c) / BS;
        scales[tiled ? tiled_scale_offset(r, j, (bpr + 7) >> 3) : r * bpr + j] =
            static_cast<uint8_t>(sc);
      }
    }
    __syncthreads();
    const int64_t col = c0 + 2 * pair;
    const int64_t row = r0 + grp * BS;
    if (col < cols && row < rows) {
#pragma unroll 1
      for (int h = 0; h < 2; ++h) {
        float v[BS];
#pragma unroll
        for (int k = 0; k < BS; ++k) {
          const uint32_t w = tile_word<BS>(tile, grp * BS + k, pair);
          v[k] = bf16_to_f32(h ? (w >> 16) : (w & 0xFFFFu));
        }
        if constexpr (RHT) rht_n(*reinterpret_cast<float(*)[16]>(v), rht, grp);
        const int64_t c = col + h;
        float amax_b = 0.0f;
#pragma unroll
        for (int k = 0; k < BS; ++k) amax_b = fmaxf(amax_b, fabsf(v[k]));
        float s_enc_l;
        const uint32_t sc =
            scale_for_block<FMT>(amax_b, s_enc_gt, s_dec_gt, s_enc_l, cnt, scale_up_t, enc_tab[1]);
        uint32_t words[BS / 8];
        encode_block<BS, RND, CNT == 2, (RHT || RRHT) ? 1 : 0>(
            v, s_enc_l, static_cast<uint64_t>(c) * rows + row, seed_t, offset_t, words, cnt);
        uint8_t* dst = codes_t + c * (rows >> 1) + (row >> 1);
        if constexpr (BS == 16) {
          *reinterpret_cast<uint2*>(dst) = make_uint2(words[0], words[1]);
        } else {
          *reinterpret_cast<uint4*>(dst) = make_uint4(words[0], words[1], words[2], words[3]);
        }
        const uint64_t kb = static_cast<uint64_t>(rows / BS);
        scales_t[tiled_t ? tiled_scale_offset(c, row / BS, (kb + 7) >> 3) : c * kb + row / BS] =
            static_cast<uint8_t>(sc);
      }
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < NB; ++k)
#pragma unroll
      for (int e = 0; e < BS / 8; ++e) q[k][e] = nq[k][e];
  }
  if constexpr (CNT) flush_counters<kThreads>(cnt, counters);
}

// ------------------------------------------------------------ 2D 16x16 --
// A workgroup covers a 64 x 64 region (4 x 4 tiles).  Thread t owns the
// 16 elements of row t/4 in tile column t%4; the 16 threads of a tile are
// lanes {c, c+4, ..., c+60} of one wave, so the tile amax is four xor
// shuffles.  Codes of W go straight out; codes of W^T go through a byte
// transpose in LDS.
// With stochastic rounding the random bits of element (r, c) are drawn at
// index r * cols + c, and the codes of W^T are the transposed codes of W,
// so both orientations hold the same rounded values (the 2D-block FP4
// page's transposition consistency, kept under SR).
template <int FMT, int RND, int CNT>
__global__ __launch_bounds__(kThreads) void k_quant_2d(
    const uint16_t* __restrict__ x, int64_t rows, int64_t cols, int64_t ld,
    uint8_t* __restrict__ codes, uint8_t* __restrict__ scales, uint8_t* __restrict__ codes_t,
    const float* __restrict__ amax, float target, float* __restrict__ s_dec_out,
    fp4_counters* __restrict__ counters, uint64_t seed, uint64_t offset, int scale_up) {
  __shared__ uint8_t tr_buf[64][64 + 4];
  float s_enc_g, s_dec_g;
  global_scales(*amax, target, s_enc_g, s_dec_g);
  if (s_dec_out && blockIdx.x == 0 && threadIdx.x == 0) *s_dec_out = s_dec_g;

  // region counts fit in 32 bits (the host keeps rows, cols below 2^31)
  const uint32_t reg_c = static_cast<uint32_t>((cols + 63) / 64);
  const uint32_t reg_r = static_cast<uint32_t>((rows + 63) / 64);
  const uint32_t nreg = reg_c * reg_r;
  const int t = threadIdx.x;
  const int lr = t >> 2, tcol = t & 3;
  uint32_t cnt[5] = {0, 0, 0, 0, 0};
  // this thread's 16 elements of region `reg` (zeros outside W or past the
  // last region: whole 16x16 tiles are in or out)
  auto load = [&](uint32_t reg, uint4 (&q)[2]) {
    const uint32_t rr = reg / reg_c, rc = reg - rr * reg_c;
    const int64_t row = static_cast<int64_t>(rr) * 64 + lr;
    const int64_t col = static_cast<int64_t>(rc) * 64 + tcol * 16;
    if (reg < nreg && row < rows && col < cols) {
      const uint4* src = reinterpret_cast<const uint4*>(x + row * ld + col);
      q[0] = src[0];
      q[1] = src[1];
    } else {
      q[0] = make_uint4(0, 0, 0, 0);
      q[1] = make_uint4(0, 0, 0, 0);
    }
  };
  uint4 q[2];
  load(blockIdx.x, q);
  for (uint32_t reg = blockIdx.x; reg < nreg; reg += gridDim.x) {
    const uint32_t rr = reg / reg_c, rc = reg - rr * reg_c;
    const int64_t r0 = static_cast<int64_t>(rr) * 64, c0 = static_cast<int64_t>(rc) * 64;
    const int64_t row = r0 + lr, col = c0 + tcol * 16;
    const bool valid = row < rows && col < cols;
    // the next region's loads are in flight while this one is encoded
    uint4 nq[2];
    load(reg + gridDim.x, nq);
    float v[16];
    unpack8(q[0], v);
    unpack8(q[1], v + 8);
    float am = 0.0f;
#pragma unroll
    for (int k = 0; k < 16; ++k) am = fmaxf(am, fabsf(v[k]));
    uint32_t amb = __float_as_uint(am);
#pragma unroll
    for (int o = 4; o < 64; o <<= 1) amb = max(amb, static_cast<uint32_t>(__shfl_xor(amb, o, 64)));
    const float amax_t = __uint_as_float(amb);
    float s_enc_l;
    uint32_t tc5[5] = {0, 0, 0, 0, 0};
    // the reciprocal is computed here, not read from a per-code table: with
    // one block per thread the table read's latency sits on the path to
    // the transposing barrier (measured slower)
    const uint32_t sc = scale_for_block<FMT>(amax_t, s_enc_g, s_dec_g, s_enc_l, tc5, scale_up);
    uint32_t words[2];
    encode_block<16, RND, CNT == 2>(v, s_enc_l, static_cast<uint64_t>(row) * cols + col, seed, offset,
                               words, cnt);
    if (valid) {
      *reinterpret_cast<uint2*>(codes + row * (cols >> 1) + (col >> 1)) =
          make_uint2(words[0], words[1]);
      if ((lr & 15) == 0) {
        scales[(row >> 4) * (cols >> 4) + (col >> 4)] = static_cast<uint8_t>(sc);
        if constexpr (CNT) {
          cnt[0] += tc5[0];
          cnt[1] += tc5[1];
          cnt[2] += tc5[2];
        }
      }
    } else if constexpr (CNT) {
      // padding lanes quantized zeros: they contribute no events
    }
    if (codes_t) {
#pragma unroll
      for (int k = 0; k < 16; ++k)
        tr_buf[tcol * 16 + k][lr] = static_cast<uint8_t>((words[k >> 3] >> (4 * (k & 7))) & 0xFu);
      __syncthreads();
      const int lc = t >> 2, rseg = (t & 3) * 16;
      const int64_t ocol = c0 + lc, orow = r0 + rseg;
      if (ocol < cols && orow < rows) {
        uint32_t w0 = 0, w1 = 0;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          w0 |= static_cast<uint32_t>(tr_buf[lc][rseg + k]) << (4 * k);
          w1 |= static_cast<uint32_t>(tr_buf[lc][rseg + 8 + k]) << (4 * k);
        }
        *reinterpret_cast<uint2*>(codes_t + ocol * (rows >> 1) + (orow >> 1)) = make_uint2(w0, w1);
      }
      __syncthreads();
    }
    q[0] = nq[0];
    q[1] = nq[1];
  }
  if constexpr (CNT) flush_counters<kThreads>(cnt, counters);
}

// ---------------------------------------------------------- dequantize --
// One thread per DQ_E consecutive values of a row of the [rows, cols] code
// matrix -- exactly one 16-byte store (8 bf16 or 4 fp32) -- so a wave's
// stores cover 1 KiB of contiguous output; kDqUnroll of them, one grid
// stride apart, are loaded before any is decoded.  The 2 (or 4, 8) threads
// of a block each read its scale byte.  sd_rows: s_dec holds one decode
// scale per row (per-row global scale).  E2M1 codes are decoded by gfx950's
// packed FP4 -> fp32 convert with a unit scale (exact: every E2M1 value is
// an fp32 value; the sign bit gives -0 for code 8), then v = (e * s_hat) *
// s_dec.
constexpr int kDqUnroll = 8;
template <bool F32>
constexpr int kDqE = F32 ? 4 : 8;

// The two E2M1 values of byte B of w, exact in fp32 (low nibble first).
template <int B>
__device__ __forceinline__ void e2m1_byte_f32(uint32_t w, float s_hat, float sd, float* v) {
  const auto e = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, B);
  v[2 * B] = (e[0] * s_hat) * sd;
  v[2 * B + 1] = (e[1] * s_hat) * sd;
}

template <int FMT, bool B2D, bool F32>
__global__ __launch_bounds__(kStream) void k_dequant(const uint8_t* __restrict__ codes,
                                                      const uint8_t* __restrict__ scales,
                                                      const float* __restrict__ s_dec,
                                                      int sd_rows, int64_t rows, int64_t cols,
                                                      void* __restrict__ out, int tiled) {
  constexpr int BS = FMT == kMX ? 32 : 16;
  constexpr int E = kDqE<F32>;                 // values per thread item
  const float sd_tensor = (FMT == kMX || sd_rows) ? 1.0f : *s_dec;
  const uint64_t ipr = static_cast<uint64_t>(cols) / E;    // items per row (cols % BS == 0)
  const uint64_t bpr = static_cast<uint64_t>(cols) / BS;
  const uint64_t n = static_cast<uint64_t>(rows) * ipr;
  const uint64_t stride = static_cast<uint64_t>(gridDim.x) * kStream;
  for (uint64_t i0 = static_cast<uint64_t>(blockIdx.x) * kStream + threadIdx.x; i0 < n;
       i0 += kDqUnroll * stride) {
    uint32_t word[kDqUnroll];
    uint32_t sc[kDqUnroll];
    float sd[kDqUnroll];
#pragma unroll
    for (int u = 0; u < kDqUnroll; ++u) {
      const uint64_t i = i0 + u * stride;
      if (i >= n) continue;
      const uint64_t r = i / ipr, j = (i - r * ipr) / (BS / E);
      sd[u] = (FMT != kMX && sd_rows) ? s_dec[r] : sd_tensor;
      sc[u] = B2D     ? scales[(r >> 4) * bpr + j]
              : tiled ? scales[tiled_scale_offset(r, j, (bpr + 7) >> 3)]
                      : scales[r * bpr + j];
      // item i's codes: bytes i * E / 2 ..
      if constexpr (F32)
        word[u] = *reinterpret_cast<const uint16_t*>(codes + i * 2);
      else
        word[u] = *reinterpret_cast<const uint32_t*>(codes + i * 4);
    }
#pragma unroll
    for (int u = 0; u < kDqUnroll; ++u) {
      const uint64_t i = i0 + u * stride;
      if (i >= n) continue;
      float s_hat;
      if constexpr (FMT == kNV) s_hat = scale_m3_decode<7>(sc[u]);
      else if constexpr (FMT == kUE) s_hat = scale_m3_decode<15>(sc[u]);
      else s_hat = ue8m0_decode(sc[u]);
      float v[E];
      e2m1_byte_f32<0>(word[u], s_hat, sd[u], v);
      e2m1_byte_f32<1>(word[u], s_hat, sd[u], v);
      if constexpr (F32) {
        *reinterpret_cast<float4*>(static_cast<float*>(out) + i * E) =
            make_float4(v[0], v[1], v[2], v[3]);
      } else {
        e2m1_byte_f32<2>(word[u], s_hat, sd[u], v);
        e2m1_byte_f32<3>(word[u], s_hat, sd[u], v);
        uint32_t hw[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          uint32_t lo = __float_as_uint(v[2 * k]), hi = __float_as_uint(v[2 * k + 1]);
          lo = (lo + 0x7FFFu + ((lo >> 16) & 1u)) >> 16;
          hi = (hi + 0x7FFFu + ((hi >> 16) & 1u)) >> 16;
          hw[k] = (lo & 0xFFFFu) | (hi << 16);
        }
        *reinterpret_cast<uint4*>(static_cast<uint16_t*>(out) + i * E) =
            make_uint4(hw[0], hw[1], hw[2], hw[3]);
      }
    }
  }
}

// ------------------------------------------------------- standalone RHT --
__global__ __launch_bounds__(kStream) void k_rht16(const uint16_t* __restrict__ x, int64_t rows,
                                                   int64_t cols, int64_t ld, uint32_t signs,
                                                   float* __restrict__ y) {
  const uint64_t pairs = static_cast<uint64_t>(cols) >> 1;
  const uint64_t n = (static_cast<uint64_t>(rows) >> 4) * pairs;
  const uint64_t stride = static_cast<uint64_t>(gridDim.x) * kStream;
  for (uint64_t i = static_cast<uint64_t>(blockIdx.x) * kStream + threadIdx.x; i < n;
       i += stride) {
    const uint64_t g = i / pairs, p = i - g * pairs;
    const uint16_t* src = x + g * 16 * ld + p * 2;
    float a[16], b[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const uint32_t w = *reinterpret_cast<const uint32_t*>(src + k * ld);
      a[k] = bf16_to_f32(w & 0xFFFFu);
      b[k] = bf16_to_f32(w >> 16);
    }
    rht16(a, signs);
    rht16(b, signs);
    float* dst = y + g * 16 * static_cast<uint64_t>(cols) + p * 2;
#pragma unroll
    for (int k = 0; k < 16; ++k)
      *reinterpret_cast<float2*>(dst + k * static_cast<uint64_t>(cols)) = make_float2(a[k], b[k]);
  }
}

// ------------------------------------------------ RHT of size N, alone --
// fl32(1/sqrt(N)) D_r H_N on every N-element group along the rows of x (N
// consecutive columns of a row), as the rowwise quantizers apply it.  One
// thread per 16-element segment; the N / 16 segments of a group are
// consecutive segments of one row, on consecutive lanes (segment s on lane
// s mod 64: the grid stride is a multiple of 64), combined by rht_n's
// shuffles.  AMX: the largest |value| goes to *amax_out (fp32 bits, atomic
// max), else the values are written to y ([rows, cols] fp32, row-major).
template <bool AMX>
__global__ __launch_bounds__(kStream) void k_rht_rows(const uint16_t* __restrict__ x, int64_t rows,
                                                      int64_t cols, int64_t ld, RhtN rht,
                                                      float* __restrict__ y,
                                                      uint32_t* __restrict__ amax_out) {
  const uint64_t seg_per_line = static_cast<uint64_t>(cols) >> 4;
  const uint64_t nseg = seg_per_line * static_cast<uint64_t>(rows);
  const uint64_t stride = static_cast<uint64_t>(gridDim.x) * kStream;
  float m = 0.0f;
  for (uint64_t sg = static_cast<uint64_t>(blockIdx.x) * kStream + threadIdx.x; sg < nseg;
       sg += stride) {
    const uint64_t line = sg / seg_per_line, j = sg - line * seg_per_line;
    float v[16];
    const uint4* src = reinterpret_cast<const uint4*>(x + line * ld + 16 * j);
    unpack8(src[0], v);
    unpack8(src[1], v + 8);
    rht_n(v, rht, static_cast<int>(threadIdx.x & 7));
    if constexpr (AMX) {
#pragma unroll
      for (int k = 0; k < 16; ++k) m = fmaxf(m, fabsf(v[k]));
    } else {
      float4* dst = reinterpret_cast<float4*>(y + line * static_cast<uint64_t>(cols) + 16 * j);
#pragma unroll
      for (int k = 0; k < 4; ++k) dst[k] = make_float4(v[4 * k], v[4 * k + 1], v[4 * k + 2], v[4 * k + 3]);
    }
  }
  if constexpr (AMX) flush_max<kStream>(__float_as_uint(m), amax_out);
}

// The RHT alone along the columns (N-row groups of each column, any N up
// to 128), written as fp32 [rows, cols].  The colwise quantizer's staging:
// a 128 x 64 tile of X goes into LDS with coalesced 16-byte row loads, each
// thread rotates one column pair of one 16-row segment (rht_n combines the
// N / 16 segments of a group across the lanes that hold them), and the
// rotated tile goes back through LDS so that every store writes whole rows.
// The row count is a multiple of N, and N divides the 128-row tile, so a
// group lies wholly inside or wholly outside the tensor.
__global__ __launch_bounds__(kThreads) void k_rht_col_tiled(const uint16_t* __restrict__ x,
                                                            int64_t rows, int64_t cols, int64_t ld,
                                                            RhtN rht, float* __restrict__ y) {
  constexpr int TR = 128, TC = 64;
  __shared__ uint4 tile[kTileChunks<16>];
  __shared__ float out_t[TR][TC + 1];
  const uint32_t tiles_c = static_cast<uint32_t>((cols + TC - 1) / TC);
  const uint32_t tiles_r = static_cast<uint32_t>((rows + TR - 1) / TR);
  const uint32_t ntiles = tiles_c * tiles_r;
  const int t = threadIdx.x;
  const int lane = t & 63, wave = t >> 6;
  const int grp = lane & 7;                  // 16-row segment of the tile
  const int pair = wave * 8 + (lane >> 3);   // column pair (0..31)
  for (uint32_t tile_id = blockIdx.x; tile_id < ntiles; tile_id += gridDim.x) {
    const uint32_t tr = tile_id / tiles_c, tc = tile_id - tr * tiles_c;
    const int64_t r0 = static_cast<int64_t>(tr) * TR, c0 = static_cast<int64_t>(tc) * TC;
#pragma unroll
    for (int k = 0; k < TR * 8 / kThreads; ++k) {
      const int chunk = t + k * kThreads;
      const int lr = chunk >> 3, lc = (chunk & 7) * 8;
      uint4 q = make_uint4(0, 0, 0, 0);
      if (r0 + lr < rows && c0 + lc < cols)
        q = *reinterpret_cast<const uint4*>(x + (r0 + lr) * ld + c0 + lc);
      tile[tile_chunk<16>(lr, chunk & 7)] = q;
    }
    __syncthreads();
    if (c0 + 2 * pair < cols && r0 + grp * 16 < rows) {
#pragma unroll 1
      for (int h = 0; h < 2; ++h) {
        float v[16];
#pragma unroll
        for (int k = 0; k < 16; ++k) {
          const uint32_t w = tile_word<16>(tile, grp * 16 + k, pair);
          v[k] = bf16_to_f32(h ? (w >> 16) : (w & 0xFFFFu));
        }
        rht_n(v, rht, grp);
#pragma unroll
        for (int k = 0; k < 16; ++k) out_t[grp * 16 + k][2 * pair + h] = v[k];
      }
    }
    __syncthreads();
    // 16 threads per 64-column tile row, 4 floats each, 16 rows per pass:
    // every store instruction writes 4 whole 256-byte row segments (the
    // LDS reads of a pass hit 64 distinct banks: rows are 65 floats apart)
    const int oc = 4 * (t & 15);
#pragma unroll
    for (int pass = 0; pass < TR / 16; ++pass) {
      const int orow = pass * 16 + (t >> 4);
      const int64_t gr = r0 + orow;
      if (gr >= rows) continue;
      float* dst = y + gr * cols + c0 + oc;
      if (c0 + oc + 4 <= cols && (reinterpret_cast<uintptr_t>(dst) & 15) == 0) {
        *reinterpret_cast<float4*>(dst) = make_float4(out_t[orow][oc], out_t[orow][oc + 1],
                                                      out_t[orow][oc + 2], out_t[orow][oc + 3]);
      } else {
        for (int e = 0; e < 4 && c0 + oc + e < cols; ++e) dst[e] = out_t[orow][oc + e];
      }
    }
  }
}

}  // namespace

namespace fp4lib {

int device_cu_count() {
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (!cache[dev]) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        n <= 0)
      n = 256;
    cache[dev] = n;
  }
  return cache[dev];
}

// Launch-geometry controls (fp4_selftest_set_geometry): results must not
// depend on them; tests vary them to expose races between waves and tiles.
static std::atomic<int> g_max_workgroups{0}, g_gemm_tile_rows{0};

void set_launch_geometry(int max_workgroups, int gemm_tile_rows) {
  g_max_workgroups.store(max_workgroups);
  g_gemm_tile_rows.store(gemm_tile_rows);
}

int64_t grid_cap(int per_cu) {
  const int64_t cap = static_cast<int64_t>(device_cu_count()) * per_cu;
  const int m = g_max_workgroups.load();
  return m > 0 && m < cap ? m : cap;
}

int gemm_tile_rows_forced() { return g_gemm_tile_rows.load(); }


hipError_t launch_amax(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld, int rht,
                       int rht_n, const uint32_t (&signs)[4], float* amax, hipStream_t s,
                       float* amax_plain, bool along_rows) {
  uint32_t* out = reinterpret_cast<uint32_t*>(amax);
  uint32_t* out_plain = reinterpret_cast<uint32_t*>(amax_plain);
  hipLaunchKernelGGL(k_fill_u32, dim3(1), dim3(1), 0, s, out, 0u);
  if (out_plain) hipLaunchKernelGGL(k_fill_u32, dim3(1), dim3(1), 0, s, out_plain, 0u);
  if (rows > 0 && cols > 0) {
    const RhtN r = make_rht(rht_n, signs);
    if (rht && along_rows) {
      // rotation along the rows (rowwise quantization): the generic kernel
      const uint64_t n = static_cast<uint64_t>(rows) * static_cast<uint64_t>(cols / 16);
      hipLaunchKernelGGL((k_rht_rows<true>), dim3(grid_for(n, kAmaxWgPerCu)), dim3(kStream),
                         0, s, x, rows, cols, ld, r, nullptr, out);
    } else if (rht && r.n == 16) {
      const uint64_t n = static_cast<uint64_t>(rows / 16) * static_cast<uint64_t>(cols / 2);
      hipLaunchKernelGGL(k_amax_rht, dim3(grid_for(n, kAmaxWgPerCu)), dim3(kStream), 0, s, x, rows, cols,
                         ld, signs[0], out, out_plain);
    } else if (rht) {
      // the other sizes: the colwise quantizer's staging and rotation, amax only
      const int64_t tiles = ((rows + 127) / 128) * ((cols + 63) / 64);
      const int64_t cap = grid_cap(kTileWgPerCu);
      const int grid = static_cast<int>(tiles < cap ? tiles : cap);
      hipLaunchKernelGGL((k_quant_col<kNV, FP4_RNE, true, 0, true>), dim3(grid),
                         dim3(kThreads), 0, s, x, rows, cols, ld, nullptr, nullptr, nullptr, 0.0f,
                         nullptr, uint64_t(0), uint64_t(0), r, nullptr, 0, out, 0);
    } else {
      const uint64_t n = static_cast<uint64_t>(rows) * static_cast<uint64_t>(cols / 8);
      hipLaunchKernelGGL(k_amax, dim3(grid_for(n, kAmaxWgPerCu)), dim3(kStream), 0, s, x, rows, cols, ld,
                         out);
    }
  }
  return hipGetLastError();
}

template <int FMT, int RND, int CNT>
static void row_launch(const QuantArgs& a, hipStream_t s) {
  constexpr int BS = FMT == kMX ? 32 : 16;
  const uint64_t n = static_cast<uint64_t>(a.rows) * static_cast<uint64_t>(a.cols / BS);
  const RhtN r = make_rht(a.rht_n, a.rht_signs);
  if constexpr (FMT != kMX) {
    if (a.rht) {
      hipLaunchKernelGGL((k_quant_row<FMT, RND, CNT, true>), dim3(grid_for(n, kRowWgPerCu)),
                         dim3(kStream), 0, s, a.x, a.rows, a.cols, a.ld, a.codes, a.scales, a.amax,
                         a.target, a.s_dec, a.seed, a.offset, a.counters, a.tiled, a.scale_up, r);
      return;
    }
  }
  hipLaunchKernelGGL((k_quant_row<FMT, RND, CNT>), dim3(grid_for(n, kRowWgPerCu)),
                     dim3(kStream), 0, s,
                     a.x, a.rows, a.cols, a.ld, a.codes, a.scales, a.amax, a.target, a.s_dec,
                     a.seed, a.offset, a.counters, a.tiled, a.scale_up, r);
}

template <int FMT, int RND>
static void row_dispatch_cnt(const QuantArgs& a, hipStream_t s) {
  if (a.counters && a.count_elems) row_launch<FMT, RND, 2>(a, s);
  else if (a.counters) row_launch<FMT, RND, 1>(a, s);
  else row_launch<FMT, RND, 0>(a, s);
}

template <int FMT>
static void row_dispatch_rnd(const QuantArgs& a, hipStream_t s) {
  if (a.round == FP4_SR) row_dispatch_cnt<FMT, FP4_SR>(a, s);
  else row_dispatch_cnt<FMT, FP4_RNE>(a, s);
}

hipError_t launch_quant_row(const QuantArgs& a, hipStream_t s) {
  if (a.format == FP4_NVFP4) row_dispatch_rnd<kNV>(a, s);
  else if (a.format == FP4_UE5M3) row_dispatch_rnd<kUE>(a, s);
  else row_dispatch_rnd<kMX>(a, s);
  return hipGetLastError();
}

template <int FMT, int RND, bool RHT, int CNT>
static void col_launch(const QuantArgs& a, hipStream_t s) {
  constexpr int BS = FMT == kMX ? 32 : 16;
  const int64_t tiles = ((a.rows + 8 * BS - 1) / (8 * BS)) * ((a.cols + 63) / 64);
  const int64_t cap = grid_cap(RND == FP4_SR ? kColWgPerCuSR : kTileWgPerCu);
  const int grid = static_cast<int>(tiles < cap ? (tiles > 0 ? tiles : 1) : cap);
  hipLaunchKernelGGL((k_quant_col<FMT, RND, RHT, CNT>), dim3(grid), dim3(kThreads), 0, s, a.x,
                     a.rows, a.cols, a.ld, a.codes, a.scales, a.amax, a.target, a.s_dec, a.seed,
                     a.offset, make_rht(a.rht_n, a.rht_signs), a.counters, a.tiled, nullptr,
                     a.scale_up);
}

template <int FMT, int RND, bool RHT>
static void col_dispatch_cnt(const QuantArgs& a, hipStream_t s) {
  if (a.counters && a.count_elems) col_launch<FMT, RND, RHT, 2>(a, s);
  else if (a.counters) col_launch<FMT, RND, RHT, 1>(a, s);
  else col_launch<FMT, RND, RHT, 0>(a, s);
}

template <int FMT, int RND>
static void col_dispatch_rht(const QuantArgs& a, hipStream_t s) {
  if constexpr (FMT == kMX) {
    col_dispatch_cnt<FMT, RND, false>(a, s);   // RHT with MXFP4 is rejected by validation
  } else {
    if (a.rht) col_dispatch_cnt<FMT, RND, true>(a, s);
    else col_dispatch_cnt<FMT, RND, false>(a, s);
  }
}

template <int FMT>
static void col_dispatch_rnd(const QuantArgs& a, hipStream_t s) {
  if (a.round == FP4_SR) col_dispatch_rht<FMT, FP4_SR>(a, s);
  else col_dispatch_rht<FMT, FP4_RNE>(a, s);
}

hipError_t launch_quant_col(const QuantArgs& a, hipStream_t s) {
  if (a.format == FP4_NVFP4) col_dispatch_rnd<kNV>(a, s);
  else if (a.format == FP4_UE5M3) col_dispatch_rnd<kUE>(a, s);
  else col_dispatch_rnd<kMX>(a, s);
  return hipGetLastError();
}

template <int FMT, int RND, bool RHT, int CNT, bool RRHT>
static void dual_launch(const QuantArgs& a, const QuantArgs& b, hipStream_t s) {
  constexpr int BS = FMT == kMX ? 32 : 16;
  const int64_t tiles = ((a.rows + 8 * BS - 1) / (8 * BS)) * ((a.cols + 63) / 64);
  const int64_t cap = grid_cap(RND == FP4_SR ? kColWgPerCuSR : kTileWgPerCu);
  const int grid = static_cast<int>(tiles < cap ? (tiles > 0 ? tiles : 1) : cap);
  hipLaunchKernelGGL((k_quant_dual<FMT, RND, RHT, CNT, RRHT>), dim3(grid), dim3(kThreads), 0, s,
                     a.x, a.rows, a.cols, a.ld, a.codes, a.scales, b.codes, b.scales, a.amax,
                     b.amax, a.target, b.target, a.s_dec, b.s_dec, a.seed, a.offset, b.seed,
                     b.offset, make_rht(b.rht_n, b.rht_signs), a.counters, a.tiled, b.tiled,
                     a.scale_up, b.scale_up, make_rht(a.rht_n, a.rht_signs));
}

template <int FMT, int RND, bool RHT>
static void dual_dispatch_cnt(const QuantArgs& a, const QuantArgs& b, hipStream_t s) {
  // the rowwise side's RHT (a.rht) only with the two-level formats
  if constexpr (FMT != kMX) {
    if (a.rht) {
      if (a.counters && a.count_elems) dual_launch<FMT, RND, RHT, 2, true>(a, b, s);
      else if (a.counters) dual_launch<FMT, RND, RHT, 1, true>(a, b, s);
      else dual_launch<FMT, RND, RHT, 0, true>(a, b, s);
      return;
    }
  }
  if (a.counters && a.count_elems) dual_launch<FMT, RND, RHT, 2, false>(a, b, s);
  else if (a.counters) dual_launch<FMT, RND, RHT, 1, false>(a, b, s);
  else dual_launch<FMT, RND, RHT, 0, false>(a, b, s);
}

template <int FMT, int RND>
static void dual_dispatch_rht(const QuantArgs& a, const QuantArgs& b, hipStream_t s) {
  if constexpr (FMT == kMX) {
    dual_dispatch_cnt<FMT, RND, false>(a, b, s);   // RHT with MXFP4 is rejected by validation
  } else {
    if (b.rht) dual_dispatch_cnt<FMT, RND, true>(a, b, s);
    else dual_dispatch_cnt<FMT, RND, false>(a, b, s);
  }
}

template <int FMT>
static void dual_dispatch_rnd(const QuantArgs& a, const QuantArgs& b, hipStream_t s) {
  if (a.round == FP4_SR) dual_dispatch_rht<FMT, FP4_SR>(a, b, s);
  else dual_dispatch_rht<FMT, FP4_RNE>(a, b, s);
}

hipError_t launch_quant_dual(const QuantArgs& row, const QuantArgs& col, hipStream_t s) {
  if (row.format == FP4_NVFP4) dual_dispatch_rnd<kNV>(row, col, s);
  else if (row.format == FP4_UE5M3) dual_dispatch_rnd<kUE>(row, col, s);
  else dual_dispatch_rnd<kMX>(row, col, s);
  return hipGetLastError();
}

template <int FMT, int RND, int CNT>
static void q2d_launch(const QuantArgs& a, hipStream_t s) {
  const int64_t regions = ((a.rows + 63) / 64) * ((a.cols + 63) / 64);
  const int64_t cap = grid_cap(kTileWgPerCu);
  const int grid = static_cast<int>(regions < cap ? (regions > 0 ? regions : 1) : cap);
  hipLaunchKernelGGL((k_quant_2d<FMT, RND, CNT>), dim3(grid), dim3(kThreads), 0, s, a.x, a.rows,
                     a.cols, a.ld, a.codes, a.scales, a.emit_transpose ? a.codes_t : nullptr,
                     a.amax, a.target, a.s_dec, a.counters, a.seed, a.offset, a.scale_up);
}

template <int FMT>
static void q2d_dispatch(const QuantArgs& a, hipStream_t s) {
  if (a.round == FP4_SR) {
    if (a.counters && a.count_elems) q2d_launch<FMT, FP4_SR, 2>(a, s);
    else if (a.counters) q2d_launch<FMT, FP4_SR, 1>(a, s);
    else q2d_launch<FMT, FP4_SR, 0>(a, s);
  } else {
    if (a.counters && a.count_elems) q2d_launch<FMT, FP4_RNE, 2>(a, s);
    else if (a.counters) q2d_launch<FMT, FP4_RNE, 1>(a, s);
    else q2d_launch<FMT, FP4_RNE, 0>(a, s);
  }
}

hipError_t launch_quant_2d(const QuantArgs& a, hipStream_t s) {
  if (a.format == FP4_NVFP4) q2d_dispatch<kNV>(a, s);
  else q2d_dispatch<kUE>(a, s);
  return hipGetLastError();
}

template <int FMT, bool B2D>
static void dq_launch(int tiled, const uint8_t* codes, const uint8_t* scales, const float* s_dec,
                      int sd_rows, int64_t rows, int64_t cols, void* out, int out_fp32,
                      hipStream_t s) {
  const int E = out_fp32 ? kDqE<true> : kDqE<false>;
  const uint64_t n = static_cast<uint64_t>(rows) * static_cast<uint64_t>(cols / E);
  const int grid = grid_for(n, 2);
  if (out_fp32)
    hipLaunchKernelGGL((k_dequant<FMT, B2D, true>), dim3(grid), dim3(kStream), 0, s, codes,
                       scales, s_dec, sd_rows, rows, cols, out, tiled);
  else
    hipLaunchKernelGGL((k_dequant<FMT, B2D, false>), dim3(grid), dim3(kStream), 0, s, codes,
                       scales, s_dec, sd_rows, rows, cols, out, tiled);
}

hipError_t launch_dequant(int format, int block2d, int tiled, const uint8_t* codes,
                          const uint8_t* scales, const float* s_dec, bool s_dec_rows,
                          int64_t rows, int64_t cols, void* out, int out_fp32, hipStream_t s) {
  const int sr = s_dec_rows ? 1 : 0;
  if (rows > 0 && cols > 0) {
    if (format == FP4_NVFP4) {
      if (block2d) dq_launch<kNV, true>(tiled, codes, scales, s_dec, sr, rows, cols, out, out_fp32, s);
      else dq_launch<kNV, false>(tiled, codes, scales, s_dec, sr, rows, cols, out, out_fp32, s);
    } else if (format == FP4_UE5M3) {
      if (block2d) dq_launch<kUE, true>(tiled, codes, scales, s_dec, sr, rows, cols, out, out_fp32, s);
      else dq_launch<kUE, false>(tiled, codes, scales, s_dec, sr, rows, cols, out, out_fp32, s);
    } else {
      dq_launch<kMX, false>(tiled, codes, scales, s_dec, 0, rows, cols, out, out_fp32, s);
    }
  }
  return hipGetLastError();
}

hipError_t launch_rht(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld, int rht_n,
                      const uint32_t (&signs)[4], bool along_rows, float* y, hipStream_t s) {
  if (rows > 0 && cols > 0) {
    const RhtN r = make_rht(rht_n, signs);
    if (!along_rows && r.n == 16) {
      const uint64_t n = static_cast<uint64_t>(rows / 16) * static_cast<uint64_t>(cols / 2);
      hipLaunchKernelGGL(k_rht16, dim3(grid_for(n, 2)), dim3(kStream), 0, s, x, rows, cols, ld,
                         signs[0], y);
    } else {
      const uint64_t n = static_cast<uint64_t>(along_rows ? rows : cols) *
                         static_cast<uint64_t>((along_rows ? cols : rows) / 16);
      if (along_rows) {
        hipLaunchKernelGGL((k_rht_rows<false>), dim3(grid_for(n, 2)), dim3(kStream), 0, s, x,
                           rows, cols, ld, r, y, nullptr);
      } else {
        const int64_t tiles = ((rows + 127) / 128) * ((cols + 63) / 64);
        const int64_t cap = grid_cap(kTileWgPerCu);
        const int grid = static_cast<int>(tiles < cap ? tiles : cap);
        hipLaunchKernelGGL(k_rht_col_tiled, dim3(grid), dim3(kThreads), 0, s, x, rows, cols, ld,
                           r, y);
      }
    }
  }
  return hipGetLastError();
}

}  // namespace fp4lib
