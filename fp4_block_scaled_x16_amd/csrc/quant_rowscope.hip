// Rowwise 1D FP4 quantizer with one global scale per row (NVFP4 paper
// App. B.1, closing remark: the global scale may span a row rather than the
// tensor, which removes the extra round trip through device memory that the
// tensor amax costs).  NVFP4 and UE5M3; RNE or stochastic rounding; with or
// without the RHT along the rows (§4.2).
//
// Each row r is quantized exactly as a one-row tensor: amax_r = max |x[r, :]|
// (over the rotated row with an RHT), s_enc_r = 6 T / amax_r, s_dec_r =
// 1 / s_enc_r (Eq. 1), then the block scales and element codes of Eqs. 2-4
// with s_enc_r, s_dec_r in place of the tensor's.
//
// Rows of up to 256 blocks (cols <= 4096): a wave owns one row at a time.
// Lane l holds blocks j = l + 64 b (b < BPT) in registers, the row amax is a
// wave reduction (no LDS, no barrier), and the next row's loads are issued
// before the current row is encoded, so every wave keeps a row in flight.
// Longer rows: a workgroup owns one row at a time, thread t holding blocks
// j = t + 256 b, the amax reduced over the four waves through LDS.  Rows of
// more than 2048 blocks (cols > 32768) are walked in chunks: a first sweep
// for the amax, then each chunk is read again and encoded (the row was read
// just before, so mostly from the L2).  Either way: one HBM read of x and no
// amax pass.
#include <hip/hip_runtime.h>

#include <stdint.h>

#include "fp4_device.hpp"
#include "fp4_internal.hpp"
#include "quant_common.hpp"

using namespace fp4dev;
using namespace fp4quant;

namespace {

constexpr int kRowThreads = 256;

// Largest |v| of one 16-element block as fp32 bits (an unsigned max of the
// magnitude bits orders finite values and infinities and keeps NaN, like
// the tensor amax kernels).  Without RHT the bf16 magnitudes are compared
// directly: fp32 bits of a bf16 value are its bits shifted left by 16.
template <bool RHT>
__device__ __forceinline__ uint32_t block_amax_bits(const uint4 (&q)[2], const RhtN& rht) {
  if constexpr (RHT) {
    float v[16];
    unpack8(q[0], v);
    unpack8(q[1], v + 8);
    rht_n(v, rht, static_cast<int>(threadIdx.x & 7));
    uint32_t m = 0;
#pragma unroll
    for (int k = 0; k < 16; ++k) m = max(m, __float_as_uint(fabsf(v[k])));
    return m;
  } else {
    const uint32_t w[8] = {q[0].x, q[0].y, q[0].z, q[0].w, q[1].x, q[1].y, q[1].z, q[1].w};
    uint32_t m = 0;
#pragma unroll
    for (int k = 0; k < 8; ++k) m = max(m, max(w[k] & 0x7FFFu, (w[k] >> 16) & 0x7FFFu));
    return m << 16;
  }
}

// Quantize the BPT blocks a lane holds (block j = j0 + stride b of row r;
// blocks at or beyond bpr are skipped) with the row's global scales.
template <int FMT, int RND, int CNT, bool RHT, int BPT>
__device__ __forceinline__ void encode_row_part(const uint4 (&q)[BPT][2], int64_t r, int64_t j0,
                                                int stride, int64_t bpr, int64_t cols,
                                                float s_enc_g, float s_dec_g, uint8_t* codes,
                                                uint8_t* scales, uint64_t kg, int tiled,
                                                int scale_up, const RhtN& rht, uint64_t seed,
                                                uint64_t offset, uint32_t (&cnt)[5]) {
  constexpr int BS = 16;
#pragma unroll
  for (int b = 0; b < BPT; ++b) {
    const int64_t j = j0 + static_cast<int64_t>(stride) * b;
    if (j >= bpr) continue;
    float v[BS];
    unpack8(q[b][0], v);
    unpack8(q[b][1], v + 8);
    if constexpr (RHT) rht_n(v, rht, static_cast<int>(threadIdx.x & 7));
    float amax_b = 0.0f;
#pragma unroll
    for (int k = 0; k < BS; ++k) amax_b = fmaxf(amax_b, fabsf(v[k]));
    float s_enc_l;
    const uint32_t sc = scale_for_block<FMT>(amax_b, s_enc_g, s_dec_g, s_enc_l, cnt, scale_up);
    uint32_t words[BS / 8];
    encode_block<BS, RND, CNT == 2>(v, s_enc_l,
                               static_cast<uint64_t>(r) * static_cast<uint64_t>(cols) +
                                   static_cast<uint64_t>(j) * BS,
                               seed, offset, words, cnt);
    *reinterpret_cast<uint2*>(codes + r * (cols >> 1) + j * (BS / 2)) =
        make_uint2(words[0], words[1]);
    scales[tiled ? tiled_scale_offset(r, j, kg) : static_cast<uint64_t>(r * bpr + j)] =
        static_cast<uint8_t>(sc);
  }
}

// Wave per row (bpr <= 64 BPT).  Same arguments as k_quant_row_scoped.
template <int FMT, int RND, int CNT, bool RHT, int BPT>
__global__ __launch_bounds__(kRowThreads) void k_quant_row_scoped_wave(
    const uint16_t* __restrict__ x, int64_t rows, int64_t cols, int64_t ld,
    uint8_t* __restrict__ codes, uint8_t* __restrict__ scales, float* __restrict__ amax,
    int amax_given, float target, float* __restrict__ s_dec_out, uint64_t seed, uint64_t offset,
    fp4_counters* __restrict__ counters, int tiled, int scale_up, RhtN rht) {
  constexpr int BS = 16;
  const int64_t bpr = cols / BS;
  const uint64_t kg = (static_cast<uint64_t>(bpr) + 7) >> 3;
  const int lane = threadIdx.x & 63;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * (kRowThreads / 64);
  uint32_t cnt[5] = {0, 0, 0, 0, 0};
  int64_t r = static_cast<int64_t>(blockIdx.x) * (kRowThreads / 64) + (threadIdx.x >> 6);
  uint4 q[BPT][2];
  auto load = [&](uint4 (&dst)[BPT][2], int64_t row) {
    const uint16_t* xr = x + row * ld;
#pragma unroll
    for (int b = 0; b < BPT; ++b) {
      const int64_t j = lane + 64 * b;
      if (j < bpr) {
        const uint4* src = reinterpret_cast<const uint4*>(xr + j * BS);
        dst[b][0] = src[0];
        dst[b][1] = src[1];
      }
    }
  };
  if (r < rows) load(q, r);
  for (; r < rows; r += stride) {
    uint4 nq[BPT][2];
    if (r + stride < rows) load(nq, r + stride);
    float row_amax;
    if (amax_given) {
      row_amax = amax[r];
    } else {
      uint32_t am = 0;
#pragma unroll
      for (int b = 0; b < BPT; ++b)
        if (lane + 64 * b < bpr) am = max(am, block_amax_bits<RHT>(q[b], rht));
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) am = max(am, static_cast<uint32_t>(__shfl_xor(am, o, 64)));
      row_amax = __uint_as_float(am);
    }
    float s_enc_g, s_dec_g;
    global_scales(row_amax, target, s_enc_g, s_dec_g);
    if (lane == 0) {
      if (!amax_given) amax[r] = row_amax;
      if (s_dec_out) s_dec_out[r] = s_dec_g;
    }
    encode_row_part<FMT, RND, CNT, RHT, BPT>(q, r, lane, 64, bpr, cols, s_enc_g, s_dec_g, codes,
                                             scales, kg, tiled, scale_up, rht, seed, offset, cnt);
#pragma unroll
    for (int b = 0; b < BPT; ++b) {
      q[b][0] = nq[b][0];
      q[b][1] = nq[b][1];
    }
  }
  if constexpr (CNT) flush_counters<kRowThreads>(cnt, counters);
}

// Workgroup per row.  BPT: 16-element blocks per thread and sweep.  amax: float[rows], read
// (amax_given) or written; s_dec_out: float[rows] or null.  The SR index of
// element (r, c) is r * cols + c, as in the tensor-scope rowwise kernel.
template <int FMT, int RND, int CNT, bool RHT, int BPT>
__global__ __launch_bounds__(kRowThreads) void k_quant_row_scoped(
    const uint16_t* __restrict__ x, int64_t rows, int64_t cols, int64_t ld,
    uint8_t* __restrict__ codes, uint8_t* __restrict__ scales, float* __restrict__ amax,
    int amax_given, float target, float* __restrict__ s_dec_out, uint64_t seed, uint64_t offset,
    fp4_counters* __restrict__ counters, int tiled, int scale_up, RhtN rht) {
  constexpr int BS = 16;
  __shared__ uint32_t red[2][kRowThreads / 64];
  const int64_t bpr = cols / BS;
  const int64_t chunk = static_cast<int64_t>(kRowThreads) * BPT;
  const bool resident = bpr <= chunk;
  const uint64_t kg = (static_cast<uint64_t>(bpr) + 7) >> 3;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t cnt[5] = {0, 0, 0, 0, 0};
  int par = 0;
  for (int64_t r = blockIdx.x; r < rows; r += gridDim.x, par ^= 1) {
    const uint16_t* xr = x + r * ld;
    uint4 q[BPT][2];
    // sweep 1: load the row (kept when it fits) and reduce its amax
    uint32_t am = 0;
    if (resident || !amax_given) {
      for (int64_t c0 = 0; c0 < bpr; c0 += chunk) {
#pragma unroll
        for (int b = 0; b < BPT; ++b) {
          const int64_t j = c0 + threadIdx.x + kRowThreads * b;
          if (j < bpr) {
            const uint4* src = reinterpret_cast<const uint4*>(xr + j * BS);
            q[b][0] = src[0];
            q[b][1] = src[1];
            if (!amax_given) am = max(am, block_amax_bits<RHT>(q[b], rht));
          }
        }
      }
    }
    float row_amax;
    if (amax_given) {
      row_amax = amax[r];
    } else {
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) am = max(am, static_cast<uint32_t>(__shfl_xor(am, o, 64)));
      if (lane == 0) red[par][wave] = am;
      __syncthreads();
      am = red[par][0];
#pragma unroll
      for (int w = 1; w < kRowThreads / 64; ++w) am = max(am, red[par][w]);
      row_amax = __uint_as_float(am);
    }
    float s_enc_g, s_dec_g;
    global_scales(row_amax, target, s_enc_g, s_dec_g);
    if (threadIdx.x == 0) {
      if (!amax_given) amax[r] = row_amax;
      if (s_dec_out) s_dec_out[r] = s_dec_g;
    }
    // sweep 2: encode (re-reading chunks of rows that did not fit)
    for (int64_t c0 = 0; c0 < bpr; c0 += chunk) {
      if (!resident) {
#pragma unroll
        for (int b = 0; b < BPT; ++b) {
          const int64_t j = c0 + threadIdx.x + kRowThreads * b;
          if (j < bpr) {
            const uint4* src = reinterpret_cast<const uint4*>(xr + j * BS);
            q[b][0] = src[0];
            q[b][1] = src[1];
          }
        }
      }
      encode_row_part<FMT, RND, CNT, RHT, BPT>(q, r, c0 + threadIdx.x, kRowThreads, bpr, cols,
                                               s_enc_g, s_dec_g, codes, scales, kg, tiled,
                                               scale_up, rht, seed, offset, cnt);
    }
  }
  if constexpr (CNT) flush_counters<kRowThreads>(cnt, counters);
}

// Persistent grid: as many workgroups as fit on the device at once (the
// kernel's occupancy, queried once per kernel), capped by the rows, so a
// wave (or workgroup) walks several rows and the wave kernel's next-row
// loads overlap the current row's encode.
template <int FMT, int RND, int CNT, bool RHT, int BPT, bool WAVE>
void scoped_launch(const fp4lib::QuantArgs& a, const RhtN& r, hipStream_t s) {
  auto kernel = WAVE ? k_quant_row_scoped_wave<FMT, RND, CNT, RHT, BPT>
                     : k_quant_row_scoped<FMT, RND, CNT, RHT, BPT>;
  static int per_cu = 0;       // benign race: every thread computes the same value
  if (per_cu == 0) {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kernel, kRowThreads, 0) != hipSuccess ||
        n < 1)
      n = 1;
    per_cu = n;
  }
  const int64_t rows_per_wg = WAVE ? kRowThreads / 64 : 1;
  const int64_t want = (a.rows + rows_per_wg - 1) / rows_per_wg;
  const int64_t cap = fp4lib::grid_cap(per_cu);
  const int grid = static_cast<int>(want < cap ? want : cap);
  hipLaunchKernelGGL(kernel, dim3(grid), dim3(kRowThreads), 0, s, a.x, a.rows, a.cols, a.ld,
                     a.codes, a.scales, const_cast<float*>(a.amax), a.amax_given, a.target,
                     a.s_dec, a.seed, a.offset, a.counters, a.tiled, a.scale_up, r);
}

// Rows of up to 256 blocks: a wave per row with the fewest of 1, 2, 4
// blocks per lane that hold it; longer rows: a workgroup per row, 2, 4 or 8
// blocks per thread (beyond 2048 blocks, in chunks of 2048).
template <int FMT, int RND, int CNT, bool RHT>
void scoped_bpt(const fp4lib::QuantArgs& a, const RhtN& r, hipStream_t s) {
  const int64_t bpr = a.cols / 16;
  if (bpr <= 64) scoped_launch<FMT, RND, CNT, RHT, 1, true>(a, r, s);
  else if (bpr <= 128) scoped_launch<FMT, RND, CNT, RHT, 2, true>(a, r, s);
  else if (bpr <= 256) scoped_launch<FMT, RND, CNT, RHT, 4, true>(a, r, s);
  else if (bpr <= 2 * kRowThreads) scoped_launch<FMT, RND, CNT, RHT, 2, false>(a, r, s);
  else if (bpr <= 4 * kRowThreads) scoped_launch<FMT, RND, CNT, RHT, 4, false>(a, r, s);
  else scoped_launch<FMT, RND, CNT, RHT, 8, false>(a, r, s);
}

template <int FMT, int RND, int CNT>
void scoped_rht(const fp4lib::QuantArgs& a, hipStream_t s) {
  const RhtN r = make_rht(a.rht_n, a.rht_signs);
  if (a.rht) scoped_bpt<FMT, RND, CNT, true>(a, r, s);
  else scoped_bpt<FMT, RND, CNT, false>(a, r, s);
}

template <int FMT>
void scoped_dispatch(const fp4lib::QuantArgs& a, hipStream_t s) {
  if (a.round == FP4_SR) {
    if (a.counters && a.count_elems) scoped_rht<FMT, FP4_SR, 2>(a, s);
    else if (a.counters) scoped_rht<FMT, FP4_SR, 1>(a, s);
    else scoped_rht<FMT, FP4_SR, 0>(a, s);
  } else {
    if (a.counters && a.count_elems) scoped_rht<FMT, FP4_RNE, 2>(a, s);
    else if (a.counters) scoped_rht<FMT, FP4_RNE, 1>(a, s);
    else scoped_rht<FMT, FP4_RNE, 0>(a, s);
  }
}

}  // namespace

namespace fp4lib {

hipError_t launch_quant_row_scoped(const QuantArgs& a, hipStream_t s) {
  // rows with no columns still get amax_r = 0 and s_dec_r = 1
  if (a.rows > 0) {
    if (a.format == FP4_NVFP4) scoped_dispatch<kNV>(a, s);
    else scoped_dispatch<kUE>(a, s);
  }
  return hipGetLastError();
}

}  // namespace fp4lib
