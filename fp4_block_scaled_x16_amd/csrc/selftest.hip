// Exhaustive device checks of the conversions on the hot path (declared in
// include/fp4_selftest.h): each kernel calls the very device functions the
// quantizers and GEMMs call and compares them with a step function or
// writes the results out; the expected values come from the caller.
//
//   k_sweep_e2m1   fp32 -> E2M1 RNE through gfx950's packed FP4 convert, two
//                  values per call into byte SEL of a word, as the quantizer
//                  packs 8 codes (NVFP4 paper §3, App. B.3 Eq. 4)
//   k_sweep_e2m1_sr  fp32 -> E2M1 by stochastic rounding (§4.4) through the
//                  quantizers' 8-value helper, with the random bits on either
//                  side of each input's carry threshold
//   k_sweep_scale  fp32 -> E4M3 / UE5M3 block-scale codes (App. B.2 Eq. 3)
//   k_sweep_e4m3_elem  fp32 -> E4M3 element codes of MXFP8 through the
//                  hardware FP8 convert, four signed values per word as the
//                  MXFP8 quantizer packs them
//   k_gemm_decode  E2M1 x block scale -> fp16, the GEMM operand decode
//                  (App. B.3)
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fp4_internal.hpp"
#include "gemm_common.hpp"

namespace {

constexpr int kSweepThreads = 256;
constexpr int kSweepWgPerCu = 4;

// Workgroup totals of (mismatches, checked) and the smallest mismatching
// pattern, then one atomic each into res[0..2].
__device__ __forceinline__ void flush_sweep(uint64_t bad, uint64_t checked, uint64_t first,
                                            unsigned long long* res) {
  __shared__ uint64_t red[kSweepThreads / 64][3];
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    bad += __shfl_xor(bad, o, 64);
    checked += __shfl_xor(checked, o, 64);
    const uint64_t f = __shfl_xor(first, o, 64);
    first = f < first ? f : first;
  }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) {
    red[wave][0] = bad;
    red[wave][1] = checked;
    red[wave][2] = first;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w = 1; w < kSweepThreads / 64; ++w) {
      bad += red[w][0];
      checked += red[w][1];
      first = red[w][2] < first ? red[w][2] : first;
    }
    if (bad) atomicAdd(&res[0], static_cast<unsigned long long>(bad));
    if (bad) atomicMin(&res[1], static_cast<unsigned long long>(first));
    atomicAdd(&res[2], static_cast<unsigned long long>(checked));
  }
}

__global__ void k_sweep_init(unsigned long long* res) {
  res[0] = 0ull;
  res[1] = ~0ull;
  res[2] = 0ull;
}

// Every fp32 pattern in groups of 8 consecutive patterns: one packed word
// per group, built by four pair converts exactly as the RNE quantizer does.
__global__ __launch_bounds__(kSweepThreads) void k_sweep_e2m1(const uint32_t* __restrict__ thr,
                                                              unsigned long long* __restrict__ res) {
  uint32_t t[7];
#pragma unroll
  for (int i = 0; i < 7; ++i) t[i] = thr[i];
  constexpr uint64_t kGroups = uint64_t(1) << 29;
  const uint64_t stride = static_cast<uint64_t>(gridDim.x) * kSweepThreads;
  uint64_t bad = 0, checked = 0, first = ~uint64_t(0);
  for (uint64_t g = static_cast<uint64_t>(blockIdx.x) * kSweepThreads + threadIdx.x; g < kGroups;
       g += stride) {
    const uint32_t b0 = static_cast<uint32_t>(g << 3);
    float y[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) y[i] = __uint_as_float(b0 + i);
    uint32_t word = 0;
    word = fp4dev::e2m1_rne_pair<0>(word, y[0], y[1]);
    word = fp4dev::e2m1_rne_pair<1>(word, y[2], y[3]);
    word = fp4dev::e2m1_rne_pair<2>(word, y[4], y[5]);
    word = fp4dev::e2m1_rne_pair<3>(word, y[6], y[7]);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t b = b0 + i;
      const uint32_t m = b & 0x7FFFFFFFu;
      if (m > 0x7F800000u) continue;   // NaN: outside the contract
      uint32_t k = 0;
#pragma unroll
      for (int j = 0; j < 7; ++j) k += m >= t[j];
      const uint32_t want = ((b >> 28) & 8u) | k;
      const uint32_t got = (word >> (4 * i)) & 0xFu;
      ++checked;
      if (got != want) {
        ++bad;
        first = b < first ? b : first;
      }
    }
  }
  flush_sweep(bad, checked, first, res);
}

// Every non-NaN fp32 pattern through the stochastic-rounding helper the
// quantizers call (e2m1_sr8).  thr holds the E2M1 magnitudes 0.5 .. 6 as fp32
// patterns: an input of magnitude m lies in [lo, hi) with lo = thr[k-1] (0
// for k = 0) and hi = thr[k], k = #(m >= thr); from the first 16 bits L of
// f = (m - lo) / (hi - lo) (fp32 arithmetic, exact here: Sterbenz, then a
// power of two) the random value 65535 - L must round down and 65536 - L
// up.  Each group of 8 patterns is converted four times: both random values,
// with the patterns in order and rotated by one place, so every pattern sits
// once at an even and once at an odd position (the two take their random
// bits from different halves of a word).  |y| >= 6 must give 6 for both.
__global__ __launch_bounds__(kSweepThreads) void k_sweep_e2m1_sr(const uint32_t* __restrict__ thr,
                                                                 unsigned long long* __restrict__ res) {
  float t[7];
#pragma unroll
  for (int i = 0; i < 7; ++i) t[i] = __uint_as_float(thr[i]);
  constexpr uint64_t kGroups = uint64_t(1) << 29;
  const uint64_t stride = static_cast<uint64_t>(gridDim.x) * kSweepThreads;
  uint64_t bad = 0, checked = 0, first = ~uint64_t(0);
  for (uint64_t g = static_cast<uint64_t>(blockIdx.x) * kSweepThreads + threadIdx.x; g < kGroups;
       g += stride) {
    const uint32_t b0 = static_cast<uint32_t>(g << 3);
#pragma unroll 1
    for (int pass = 0; pass < 4; ++pass) {
      const int rot = pass >> 1, up_side = pass & 1;
      float y[8];
      uint32_t pat[8], want[8], u[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        pat[i] = b0 + static_cast<uint32_t>((i + rot) & 7);
        y[i] = __uint_as_float(pat[i]);
        const float m = __uint_as_float(pat[i] & 0x7FFFFFFFu);
        uint32_t k = 0;
#pragma unroll
        for (int j = 0; j < 7; ++j) k += m >= t[j] ? 1u : 0u;
        uint32_t mag = 7u;
        u[i] = up_side ? 65535u : 0u;
        if (k < 7u) {
          const float lo = k ? t[k > 0 ? k - 1 : 0] : 0.0f;
          const float hi = t[k];
          const uint32_t lead = static_cast<uint32_t>((m - lo) / (hi - lo) * 65536.0f);
          // lead = 0: no random value rounds up; test 65535 on both sides
          u[i] = (up_side && lead) ? 65536u - lead : 65535u - (lead ? lead : 0u);
          mag = k + ((u[i] + lead >= 65536u) ? 1u : 0u);
        }
        want[i] = ((pat[i] >> 28) & 8u) | mag;
      }
      const fp4dev::U4 w{(u[0] << 16) | u[1], (u[2] << 16) | u[3], (u[4] << 16) | u[5],
                         (u[6] << 16) | u[7]};
      const uint32_t word = fp4dev::e2m1_sr8(y, w);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        if ((pat[i] & 0x7FFFFFFFu) > 0x7F800000u) continue;   // NaN: outside the contract
        ++checked;
        if (((word >> (4 * i)) & 0xFu) != want[i]) {
          ++bad;
          first = pat[i] < first ? pat[i] : first;
        }
      }
    }
  }
  flush_sweep(bad, checked, first, res);
}

// Every finite fp32 t >= 0 through the block-scale encoder; the expected
// code is the number of thresholds <= t (binary search over 256 entries,
// padded with patterns above every input).
template <int BIAS>
__global__ __launch_bounds__(kSweepThreads) void k_sweep_scale(const uint32_t* __restrict__ thr,
                                                               int n,
                                                               unsigned long long* __restrict__ res) {
  __shared__ uint32_t t[256];
  t[threadIdx.x] = static_cast<int>(threadIdx.x) < n ? thr[threadIdx.x] : 0xFFFFFFFFu;
  __syncthreads();
  constexpr uint64_t kEnd = 0x7F800000ull;   // first non-finite pattern
  const uint64_t stride = static_cast<uint64_t>(gridDim.x) * kSweepThreads;
  uint64_t bad = 0, checked = 0, first = ~uint64_t(0);
  for (uint64_t b = static_cast<uint64_t>(blockIdx.x) * kSweepThreads + threadIdx.x; b < kEnd;
       b += stride) {
    const float tv = __uint_as_float(static_cast<uint32_t>(b));
    const uint32_t got = BIAS == 7 ? fp4dev::scale_m3_encode<7>(tv, 448.0f, 0x7Eu)
                                   : fp4dev::scale_m3_encode<15>(tv, 122880.0f, 0xFFu);
    uint32_t pos = 0;
#pragma unroll
    for (uint32_t s = 128; s >= 1; s >>= 1)
      if (t[pos + s - 1] <= static_cast<uint32_t>(b)) pos += s;
    ++checked;
    if (got != pos) {
      ++bad;
      first = b < first ? b : first;
    }
  }
  flush_sweep(bad, checked, first, res);
}

// Every fp32 magnitude t in [0, 448] through the MXFP8 element packer, as
// (t, -t, -t, t) and (-t, t, t, -t): each byte position with either sign.
// Expected magnitude code: the number of thresholds <= t, sign in bit 7.
__global__ __launch_bounds__(kSweepThreads) void k_sweep_e4m3_elem(const uint32_t* __restrict__ thr,
                                                                   int n,
                                                                   unsigned long long* __restrict__ res) {
  __shared__ uint32_t t[256];
  t[threadIdx.x] = static_cast<int>(threadIdx.x) < n ? thr[threadIdx.x] : 0xFFFFFFFFu;
  __syncthreads();
  constexpr uint64_t kEnd = 0x43E00001ull;   // one past 448.0f
  const uint64_t stride = static_cast<uint64_t>(gridDim.x) * kSweepThreads;
  uint64_t bad = 0, checked = 0, first = ~uint64_t(0);
  for (uint64_t b = static_cast<uint64_t>(blockIdx.x) * kSweepThreads + threadIdx.x; b < kEnd;
       b += stride) {
    const float tv = __uint_as_float(static_cast<uint32_t>(b));
    const uint32_t w0 = fp4dev::e4m3_pack4(tv, -tv, -tv, tv);
    const uint32_t w1 = fp4dev::e4m3_pack4(-tv, tv, tv, -tv);
    uint32_t pos = 0;
#pragma unroll
    for (uint32_t s = 128; s >= 1; s >>= 1)
      if (t[pos + s - 1] <= static_cast<uint32_t>(b)) pos += s;
    const uint32_t ng = pos | 0x80u;
    const uint32_t e0 = pos | (ng << 8) | (ng << 16) | (pos << 24);
    const uint32_t e1 = ng | (pos << 8) | (pos << 16) | (ng << 24);
    ++checked;
    if (w0 != e0 || w1 != e1) {
      ++bad;
      first = b < first ? b : first;
    }
  }
  flush_sweep(bad, checked, first, res);
}

// One thread per block-scale code s: the 16 E2M1 codes times s, with s in
// the low and then in the high half of the scale pair, the pair taken from
// bytes 0-1 and then from bytes 2-3 of a word.
// The code words are made from `salt` (0 at run time) so that, as in the
// GEMM, they are run-time values in vector registers; the fp16 results are
// stored as whole 8-element vectors (element-wise stores through
// __builtin_bit_cast of vector elements lost all but element 0 of each
// vector under -O3).
template <int FMT>
__global__ __launch_bounds__(256) void k_gemm_decode(uint16_t* __restrict__ out, uint32_t salt) {
  using namespace fp4gemm;
  const uint32_t s = threadIdx.x;
  constexpr uint32_t kCodes = FMT == kNV ? 0x7Fu : 256u;
  uint16_t* o = out + s * 64;
  if (s >= kCodes) {
#pragma unroll
    for (int i = 0; i < 64; ++i) o[i] = 0;
    return;
  }
  const uint32_t other = (s + 1u + (s * 37u) % (kCodes - 1u)) % kCodes;   // != s
  const uint32_t lo = 0x76543210u ^ (salt * s), hi = 0xFEDCBA98u ^ (salt * s);
  // the scale pair from bytes 0-1 of a word (bytes 2-3 hold other codes),
  // then from bytes 2-3
  const uint32_t w0 = s | (other << 8) | ((other ^ 0x55u) % kCodes << 16);
  const uint32_t w1 = other | (s << 8) | ((other ^ 0x2Au) % kCodes << 24);
  half8 v[8];
  uint32_t pair = scale_pair_f16<FMT, 0>(w0);
  v[0] = dequant8<0>(lo, pair);
  v[1] = dequant8<0>(hi, pair);
  pair = scale_pair_f16<FMT, 0>(w1);
  v[2] = dequant8<1>(lo, pair);
  v[3] = dequant8<1>(hi, pair);
  pair = scale_pair_f16<FMT, 2>((w0 << 16) | ((other ^ 0x33u) % kCodes));
  v[4] = dequant8<0>(lo, pair);
  v[5] = dequant8<0>(hi, pair);
  pair = scale_pair_f16<FMT, 2>((w1 << 16) | ((other ^ 0x66u) % kCodes << 8));
  v[6] = dequant8<1>(lo, pair);
  v[7] = dequant8<1>(hi, pair);
#pragma unroll
  for (int q = 0; q < 8; ++q) *reinterpret_cast<half8*>(o + 8 * q) = v[q];   // 16-byte aligned
}

}  // namespace

namespace fp4lib {

hipError_t launch_selftest_sweep(int kind, const uint32_t* thresholds, int n, uint64_t* result,
                                 hipStream_t s) {
  auto* res = reinterpret_cast<unsigned long long*>(result);
  hipLaunchKernelGGL(k_sweep_init, dim3(1), dim3(1), 0, s, res);
  const int grid = device_cu_count() * kSweepWgPerCu;
  if (kind == FP4_SWEEP_E2M1_RNE)
    hipLaunchKernelGGL(k_sweep_e2m1, dim3(grid), dim3(kSweepThreads), 0, s, thresholds, res);
  else if (kind == FP4_SWEEP_E2M1_SR)
    hipLaunchKernelGGL(k_sweep_e2m1_sr, dim3(grid), dim3(kSweepThreads), 0, s, thresholds, res);
  else if (kind == FP4_SWEEP_E4M3_SCALE)
    hipLaunchKernelGGL(k_sweep_scale<7>, dim3(grid), dim3(kSweepThreads), 0, s, thresholds, n, res);
  else if (kind == FP4_SWEEP_E4M3_ELEM)
    hipLaunchKernelGGL(k_sweep_e4m3_elem, dim3(grid), dim3(kSweepThreads), 0, s, thresholds, n,
                       res);
  else
    hipLaunchKernelGGL(k_sweep_scale<15>, dim3(grid), dim3(kSweepThreads), 0, s, thresholds, n,
                       res);
  return hipGetLastError();
}

hipError_t launch_selftest_gemm_decode(int format, uint16_t* out, hipStream_t s) {
  if (format == FP4_NVFP4)
    hipLaunchKernelGGL(k_gemm_decode<fp4dev::kNV>, dim3(1), dim3(256), 0, s, out, 0u);
  else
    hipLaunchKernelGGL(k_gemm_decode<fp4dev::kUE>, dim3(1), dim3(256), 0, s, out, 0u);
  return hipGetLastError();
}

}  // namespace fp4lib
