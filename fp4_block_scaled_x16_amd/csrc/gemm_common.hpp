// Shared pieces of the block-scaled FP4 GEMM kernels: the launch
// parameters, tile order, epilogue, LDS swizzle and wait helpers, and the
// NVFP4 / UE5M3 dequantize-and-multiply slice.  Each kernel family lives in
// its own translation unit (gemm_nv.hip, gemm_nv_dma.hip -- built once per
// format and tile height --, gemm_mx.hip, gemm_mx_dma.hip) behind the launch
// functions declared at the end; the dispatch between them is in gemm.hip.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fp4_device.hpp"
#include "fp4_internal.hpp"

using namespace fp4dev;


namespace fp4gemm {


typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef int int8v __attribute__((ext_vector_type(8)));

constexpr int kBM = 256, kBN = 256, kThreads = 256;

struct Params {
  const uint8_t* codes[2];
  int64_t ld[2];
  const uint8_t* scales[2];
  int64_t s_row[2], s_kblk[2];
  int rg_shift[2];      // log2 of the scale row group (0 or 4)
  const float* s_dec[2];
  int s_dec_rows[2];    // s_dec holds one decode scale per operand row (per-row global scale)
  float* D;             // fp32, or bf16 (d_bf16) reinterpreted; ldd in elements
  int d_bf16;
  int64_t ldd;
  int64_t M, N, K;
  int accumulate;
  int tiles_m, tiles_n;
  int vec16[2];         // code rows are 16-byte aligned
  int sc_vec[2];        // the scales of one row and K step are contiguous and aligned
  int tiled[2];         // scales in the TILED layout (s_row unused, s_kblk = 1)
  int64_t kg;           // TILED: atoms (8 K-blocks each) per 256-row band
};

// Scales of row `row`, K-blocks kb0, kb0 + 1, ... at stride p.s_kblk[o]
// (1 in the TILED layout, where the 4 or 8 blocks of a K step share an atom).
__device__ __forceinline__ const uint8_t* scale_ptr(const Params& p, int o, int64_t row,
                                                    int64_t kb0) {
  if (p.tiled[o]) return p.scales[o] + tiled_scale_offset(row, kb0, p.kg);
  return p.scales[o] + (row >> p.rg_shift[o]) * p.s_row[o] + kb0 * p.s_kblk[o];
}

// Tile order: consecutive workgroup ids go round-robin over the 8 XCDs, so
// first give each XCD a contiguous range of tiles, then walk that range in
// groups of 8 tile-rows so neighbouring tiles share A rows and B columns in
// the XCD's L2.
__device__ __forceinline__ void tile_coords(const Params& p, int& tm, int& tn) {
  const int T = p.tiles_m * p.tiles_n;
  int id = blockIdx.x;
  if ((T & 7) == 0) id = (id & 7) * (T >> 3) + (id >> 3);
  constexpr int G = 8;
  const int per_group = G * p.tiles_n;
  const int g = id / per_group;
  const int first = g * G;
  const int gm = min(p.tiles_m - first, G);
  const int r = id - g * per_group;
  tm = first + r % gm;
  tn = r / gm;
}

// 16 bytes of codes at byte offset `off` of a row of `row_bytes` valid
// bytes; K is a multiple of 16 so a chunk is full, half (8 bytes) or empty.
// Rows whose stride is only 8-byte aligned are read as two 8-byte halves.
__device__ __forceinline__ uint4 load_codes16(const uint8_t* row, int64_t off, int64_t row_bytes,
                                              bool vec16) {
  const int64_t left = row_bytes - off;
  if (vec16 && left >= 16) return *reinterpret_cast<const uint4*>(row + off);
  uint2 lo = make_uint2(0u, 0u), hi = make_uint2(0u, 0u);
  if (left >= 8) lo = *reinterpret_cast<const uint2*>(row + off);
  if (left >= 16) hi = *reinterpret_cast<const uint2*>(row + off + 8);
  return make_uint4(lo.x, lo.y, hi.x, hi.y);
}

// The MFMAs are issued as C^T = B A^T (B fragment in the "A" slot), so the
// 16 accumulators of a lane hold one output row m and, for each group g of
// 4, the 4 consecutive columns 8g + 4h .. +3 of a 32 x 32 tile: the
// epilogue writes 16 bytes per store.
// MI 32-row MFMA tiles per wave in M (a wave covers MI * 32 rows).
// fp32 -> bf16, round to nearest even; NaN stays a (quiet) NaN.
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float v) {
  const uint32_t u = __float_as_uint(v);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (u >> 16) | 0x40u;
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// The store loop of `epilogue` for a bf16 D (NVFP4 paper §4.1: the GEMMs
// may write BF16): each value is formed in fp32 exactly as for an fp32 D
// (with accumulate: the old bf16 value widened and added in fp32), then
// rounded once to bf16; 8 bytes per store.
template <int MI>
__device__ __forceinline__ void epilogue_bf16(const Params& p, floatx16 (&acc)[MI][4],
                                              float scale, int64_t m0, int64_t n0, int wm,
                                              int wn, int lane) {
  const int i = lane & 31, h = lane >> 5;
  uint16_t* d16 = reinterpret_cast<uint16_t*>(p.D);
  const bool vec = (p.ldd & 3) == 0 && (reinterpret_cast<uintptr_t>(d16) & 7) == 0;
#pragma unroll
  for (int mi = 0; mi < MI; ++mi) {
    const int64_t row = m0 + wm * (MI * 32) + mi * 32 + i;
    if (row >= p.M) continue;
    uint16_t* drow = d16 + row * p.ldd;
#pragma unroll
    for (int ni = 0; ni < 4; ++ni) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int64_t col = n0 + wn * 128 + ni * 32 + 8 * g + 4 * h;
        float r[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) r[e] = acc[mi][ni][4 * g + e] * scale;
        if (vec && col + 3 < p.N) {
          uint2* dst = reinterpret_cast<uint2*>(drow + col);
          if (p.accumulate) {
            const uint2 o = *dst;
            r[0] += __uint_as_float(o.x << 16);
            r[1] += __uint_as_float(o.x & 0xFFFF0000u);
            r[2] += __uint_as_float(o.y << 16);
            r[3] += __uint_as_float(o.y & 0xFFFF0000u);
          }
          *dst = make_uint2(f32_to_bf16_rne(r[0]) | (f32_to_bf16_rne(r[1]) << 16),
                            f32_to_bf16_rne(r[2]) | (f32_to_bf16_rne(r[3]) << 16));
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            if (col + e < p.N) {
              uint16_t* d = drow + col + e;
              const float v = p.accumulate ? r[e] + __uint_as_float(uint32_t(*d) << 16) : r[e];
              *d = static_cast<uint16_t>(f32_to_bf16_rne(v));
            }
          }
        }
      }
    }
  }
}

// Epilogue through LDS, for a wave whose whole MI * 32 x 128 part of the
// tile lies inside D, with no per-row decode scales.  In the MFMA output
// layout lane (i, h) holds row i, columns 8g + 4h .. + 3 (g = 0..3) of a
// 32 x 32 block, so a plain 16-byte store covers 32 rows with 32 bytes
// each (and a bf16 one 32 rows with 16 bytes).  Here each block goes
// through a per-wave LDS buffer of 32 rows x kEpiPitch floats and comes out
// with 8 consecutive lanes holding one row's 32 values, so every store
// writes 8 whole 128-byte row segments (a bf16 D: 8 rows x 64 bytes) -- 4x
// fewer memory requests; the D write was the larger part of the epilogue.
// The pitch of 36 floats puts the rows one write pass covers, and the 2
// rows one read pass covers, on different banks.  Values are (acc * pre) *
// scale in fp32 -- the same two roundings as multiplying the accumulators
// by `pre` and calling `epilogue` with `scale` -- plus the old D (fp32,
// accumulate), or rounded once to bf16 (no accumulation).  ALL: also the
// accumulate and bf16 cases; without it only a plain fp32 D (the 256-row
// kernels have no registers to spare for the other two: with them the
// compiler spilled values of every path, the plain one included).
constexpr int kEpiPitch = 36;
constexpr int kEpiBufFloats = 32 * kEpiPitch;

template <int MI, bool ALL>
__device__ __forceinline__ bool epilogue_lds_ok(const Params& p, int64_t m0, int64_t n0, int wm,
                                                int wn) {
  if (!ALL && (p.d_bf16 || p.accumulate)) return false;
  // rows of D 16-byte (fp32) or 8-byte (bf16) aligned
  return !p.s_dec_rows[0] && !p.s_dec_rows[1] && !(p.d_bf16 && p.accumulate) &&
         (p.ldd & 3) == 0 && (reinterpret_cast<uintptr_t>(p.D) & 15) == 0 &&
         m0 + wm * (MI * 32) + MI * 32 <= p.M && n0 + wn * 128 + 128 <= p.N;
}

// 32 x 32 fp32 block through `buf`: v[r] = this lane's 4 values of row
// 8r + lane / 8, columns 4 (lane % 8) .. + 3, unscaled (the accumulators go
// out straight from their registers; the scaling is per element, so the
// caller applies it after the transpose).
__device__ __forceinline__ void lds_transpose_f32(const floatx16& a, float* buf, int lane,
                                                  float4 (&v)[4]) {
  const int i = lane & 31, h = lane >> 5;
#pragma unroll
  for (int g = 0; g < 4; ++g)
    *reinterpret_cast<float4*>(buf + i * kEpiPitch + 8 * g + 4 * h) =
        make_float4(a[4 * g], a[4 * g + 1], a[4 * g + 2], a[4 * g + 3]);
  // the other lanes' writes are read next: order them within the wave
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
#pragma unroll
  for (int r = 0; r < 4; ++r)
    v[r] = *reinterpret_cast<const float4*>(buf + (8 * r + (lane >> 3)) * kEpiPitch +
                                            4 * (lane & 7));
  // and these reads precede the next writes into the buffer
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
}

__device__ __forceinline__ float4 scale4(const float4& v, float pre, float scale) {
  return make_float4((v.x * pre) * scale, (v.y * pre) * scale, (v.z * pre) * scale,
                     (v.w * pre) * scale);
}

// lds_t: this wave's BUFS * kEpiBufFloats words (with 2, consecutive blocks
// alternate halves).
template <int MI, int BUFS, bool ALL>
__device__ __forceinline__ void epilogue_lds(const Params& p, floatx16 (&acc)[MI][4], float pre,
                                             float scale, int64_t m0, int64_t n0, int wm, int wn,
                                             int lane, float* lds_t) {
  const int lr = lane >> 3, lc = lane & 7;    // row within 8, 16-byte chunk within 128 bytes
  const int64_t wr0 = m0 + wm * (MI * 32), wc0 = n0 + wn * 128;
  // one straight-line loop per case (a branch per block on the case costs
  // the plain fp32 loop measurably)
  if (ALL && p.accumulate) {
    // the old D of a block is loaded ahead of its LDS round trip, in the
    // same coalesced layout as the stores
#pragma unroll
    for (int mi = 0; mi < MI; ++mi) {
#pragma unroll
      for (int ni = 0; ni < 4; ++ni) {
        const int64_t row0 = wr0 + mi * 32, col0 = wc0 + ni * 32;
        float4 old[4];
#pragma unroll
        for (int r = 0; r < 4; ++r)
          old[r] = *reinterpret_cast<const float4*>(p.D + (row0 + 8 * r + lr) * p.ldd + col0 +
                                                    4 * lc);
        float4 v[4];
        lds_transpose_f32(acc[mi][ni],
                          lds_t + (BUFS == 2 ? ((mi * 4 + ni) & 1) * kEpiBufFloats : 0), lane, v);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float4 y = scale4(v[r], pre, scale);
          *reinterpret_cast<float4*>(p.D + (row0 + 8 * r + lr) * p.ldd + col0 + 4 * lc) =
              make_float4(y.x + old[r].x, y.y + old[r].y, y.z + old[r].z, y.w + old[r].w);
        }
      }
    }
    return;
  }
  if (ALL && p.d_bf16) {
    // 8 lanes write a row's 64 bytes
    uint16_t* d16 = reinterpret_cast<uint16_t*>(p.D);
#pragma unroll
    for (int mi = 0; mi < MI; ++mi) {
#pragma unroll
      for (int ni = 0; ni < 4; ++ni) {
        const int64_t row0 = wr0 + mi * 32, col0 = wc0 + ni * 32;
        float4 v[4];
        lds_transpose_f32(acc[mi][ni],
                          lds_t + (BUFS == 2 ? ((mi * 4 + ni) & 1) * kEpiBufFloats : 0), lane, v);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float4 y = scale4(v[r], pre, scale);
          *reinterpret_cast<uint2*>(d16 + (row0 + 8 * r + lr) * p.ldd + col0 + 4 * lc) =
              make_uint2(f32_to_bf16_rne(y.x) | (f32_to_bf16_rne(y.y) << 16),
                         f32_to_bf16_rne(y.z) | (f32_to_bf16_rne(y.w) << 16));
        }
      }
    }
    return;
  }
#pragma unroll
  for (int mi = 0; mi < MI; ++mi) {
#pragma unroll
    for (int ni = 0; ni < 4; ++ni) {
      const int64_t row0 = wr0 + mi * 32, col0 = wc0 + ni * 32;
      float4 v[4];
      lds_transpose_f32(acc[mi][ni],
                        lds_t + (BUFS == 2 ? ((mi * 4 + ni) & 1) * kEpiBufFloats : 0), lane, v);
#pragma unroll
      for (int r = 0; r < 4; ++r)
        *reinterpret_cast<float4*>(p.D + (row0 + 8 * r + lr) * p.ldd + col0 + 4 * lc) =
            scale4(v[r], pre, scale);
    }
  }
}

// `scale` is the tensor-level s_dec_B (1 when B has per-row scales).  Per-row
// decode scales (s_dec_A[m], s_dec_B[n]) are multiplied into the
// accumulators before the first store: either read from LDS copies of the
// tile's scales (lds_a / lds_b, indexed by the row or column within the
// tile), or loaded from global memory ahead of every store (a wait for a
// load issued between stores would wait for those stores too).
template <int MI>
__device__ __forceinline__ void epilogue(const Params& p, floatx16 (&acc)[MI][4], float scale,
                                         int64_t m0, int64_t n0, int wm, int wn, int lane,
                                         const float* lds_a = nullptr,
                                         const float* lds_b = nullptr) {
  const int i = lane & 31, h = lane >> 5;
  const bool vec = (p.ldd & 3) == 0 && (reinterpret_cast<uintptr_t>(p.D) & 15) == 0;
  if (p.s_dec_rows[0]) {
    float sa[MI];
#pragma unroll
    for (int mi = 0; mi < MI; ++mi) {
      const int lr = wm * (MI * 32) + mi * 32 + i;
      const int64_t row = m0 + lr;
      sa[mi] = lds_a ? lds_a[lr] : row < p.M ? p.s_dec[0][row] : 1.0f;
    }
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
      for (int ni = 0; ni < 4; ++ni) acc[mi][ni] *= sa[mi];
  }
  if (p.s_dec_rows[1]) {
    const bool vec_b = (reinterpret_cast<uintptr_t>(p.s_dec[1]) & 15) == 0;
    float cb[4][16];
#pragma unroll
    for (int ni = 0; ni < 4; ++ni) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int lc = wn * 128 + ni * 32 + 8 * g + 4 * h;
        const int64_t col = n0 + lc;
        if (lds_b) {
          const float4 t = *reinterpret_cast<const float4*>(lds_b + lc);
          cb[ni][4 * g] = t.x;
          cb[ni][4 * g + 1] = t.y;
          cb[ni][4 * g + 2] = t.z;
          cb[ni][4 * g + 3] = t.w;
        } else if (vec_b && col + 3 < p.N) {
          const float4 t = *reinterpret_cast<const float4*>(p.s_dec[1] + col);
          cb[ni][4 * g] = t.x;
          cb[ni][4 * g + 1] = t.y;
          cb[ni][4 * g + 2] = t.z;
          cb[ni][4 * g + 3] = t.w;
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            cb[ni][4 * g + e] = col + e < p.N ? p.s_dec[1][col + e] : 1.0f;
        }
      }
    }
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
      for (int ni = 0; ni < 4; ++ni)
#pragma unroll
        for (int k = 0; k < 16; ++k) acc[mi][ni][k] *= cb[ni][k];
  }
  if (p.d_bf16) {
    epilogue_bf16(p, acc, scale, m0, n0, wm, wn, lane);
    return;
  }
#pragma unroll
  for (int mi = 0; mi < MI; ++mi) {
    const int64_t row = m0 + wm * (MI * 32) + mi * 32 + i;
    if (row >= p.M) continue;
    float* drow = p.D + row * p.ldd;
#pragma unroll
    for (int ni = 0; ni < 4; ++ni) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int64_t col = n0 + wn * 128 + ni * 32 + 8 * g + 4 * h;
        float r[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) r[e] = acc[mi][ni][4 * g + e] * scale;
        if (vec && col + 3 < p.N) {
          float4* dst = reinterpret_cast<float4*>(drow + col);
          if (p.accumulate) {
            const float4 o = *dst;
            r[0] += o.x;
            r[1] += o.y;
            r[2] += o.z;
            r[3] += o.w;
          }
          *dst = make_float4(r[0], r[1], r[2], r[3]);
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            if (col + e < p.N) {
              float* d = drow + col + e;
              *d = p.accumulate ? *d + r[e] : r[e];
            }
          }
        }
      }
    }
  }
}

constexpr int kBKX = 128;   // K per step: 64 code bytes and 4 E8M0 scales per row
constexpr int kStagesX = 4;   // MXFP4 DMA ring: stages of one K step each

// The 16-byte chunk q of LDS row r lives at position q ^ dma_swizzle(r):
// 8 (or 16) consecutive rows reading the same chunk hit distinct banks.
__device__ __forceinline__ int dma_swizzle(int row) { return ((row >> 1) ^ (row >> 2)) & 3; }

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Workgroup barrier without the release/acquire fences of __syncthreads
// (those would also drain the DMA ring): this wave's LDS reads are complete
// (lgkmcnt 0) and the compiler may move no memory access across it.
__device__ __forceinline__ void ring_barrier() {
  __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4));
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}


// ------------------------------------------------------- NVFP4 / UE5M3 --
constexpr int kBK2 = 128;   // K per step: 64 code bytes and 8 scales per row

typedef unsigned short ushort2v __attribute__((ext_vector_type(2)));

// Two consecutive block scales (codes in bytes B and B + 1 of `word`) as an
// fp16 pair, block 2k in the low half.  E4M3 uses the packed hardware FP8 ->
// fp16 convert with a unit scale (exact: every E4M3 value, subnormals
// included, is an fp16 value).  UE5M3 (bias 15, like fp16) shifted left by 7
// is bit for bit the fp16 of its value, subnormals included, for every code
// but those with exponent field 31 (fp16 infinities / NaNs).  Times 2^-5:
// the fp16 multiply is exact for exponent fields up to 30; the integer
// exponent decrement max(h, 6 << 10) - (5 << 10) is exact from 6 up (31
// included) and gives 2^-14 below, more than any product there; so the
// unsigned minimum of the two is exact for every code (at 31 the multiply
// gives an infinity or NaN, above 0x7C00).  Checked on all 256 codes.
template <int FMT, int B = 0>
__device__ __forceinline__ uint32_t scale_pair_f16(uint32_t word) {
  static_assert(B == 0 || B == 2, "a pair starts at byte 0 or 2");
  if constexpr (FMT == kNV) {
    return __builtin_bit_cast(uint32_t,
                              __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(word, 1.0f, B == 2));
  } else {
    // bytes B, B + 1 -> the low bytes of the two halves (0x0C selects zero)
    constexpr uint32_t kSel = B == 0 ? 0x0C010C00u : 0x0C030C02u;
    const ushort2v h = __builtin_bit_cast(ushort2v, __builtin_amdgcn_perm(0u, word, kSel)) << 7;
    const ushort2v dec = __builtin_elementwise_max(h, ushort2v{0x1800, 0x1800}) -
                         ushort2v{0x1400, 0x1400};
    const half2v mul = __builtin_bit_cast(half2v, h) * half2v{0x1p-5f16, 0x1p-5f16};
    return __builtin_bit_cast(uint32_t,
                              __builtin_elementwise_min(dec, __builtin_bit_cast(ushort2v, mul)));
  }
}

// Eight E2M1 codes times one block scale (exact in fp16): the scale is one
// half of an fp16 pair, broadcast by the packed multiply's operand select.
template <int HALF>
__device__ __forceinline__ half8 dequant8(uint32_t codes, uint32_t pair) {
  const half2v sp = __builtin_bit_cast(half2v, pair);
  const half2v s = HALF ? half2v{sp[1], sp[1]} : half2v{sp[0], sp[0]};
  half2v p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 0);
  half2v p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 1);
  half2v p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 2);
  half2v p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 3);
  p0 *= s;
  p1 *= s;
  p2 *= s;
  p3 *= s;
  return half8{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

struct Stage2 {
  // codes: [operand][chunk q 0..3][row slot][16 B], slot = row ^ (q << 2)
  uint4 codes[2][4][256];
  // scales: [operand][half h][row] -> fp16 pairs of blocks 4h..4h+3 of the step
  uint2 scales[2][2][256];
};

// Fragments of one MFMA K slice (16 K-values): lane half h holds the slice's
// 8 K-values of its row for each of the wave's MI A and 4 B tiles.
template <int MI>
struct FragT {
  half8 a[MI], b[4];
};
using Frag = FragT<4>;

template <int KS, int MI>
__device__ __forceinline__ void dequant_slice(FragT<MI>& f, const uint32_t (&a_raw)[MI][8],
                                              const uint32_t (&b_raw)[4][8], const uint2 (&a_sc)[MI],
                                              const uint2 (&b_sc)[4]) {
  constexpr int W = KS >> 1;     // block of the lane's 4: one 16-element block per two slices
#pragma unroll
  for (int mi = 0; mi < MI; ++mi)
    f.a[mi] = dequant8<W & 1>(a_raw[mi][KS], (W >> 1) ? a_sc[mi].y : a_sc[mi].x);
#pragma unroll
  for (int ni = 0; ni < 4; ++ni)
    f.b[ni] = dequant8<W & 1>(b_raw[ni][KS], (W >> 1) ? b_sc[ni].y : b_sc[ni].x);
}

template <int MI>
__device__ __forceinline__ void mfma_slice(floatx16 (&acc)[MI][4], const FragT<MI>& f) {
#pragma unroll
  for (int mi = 0; mi < MI; ++mi)
#pragma unroll
    for (int ni = 0; ni < 4; ++ni)
      acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_f16(f.b[ni], f.a[mi], acc[mi][ni], 0, 0, 0);
}

// Scheduling hint for one slice: alternate one MFMA with the VALU ops of
// the next slice's dequantization (8 per tile, (MI + 4) tiles over 4 MI
// MFMAs: 4 per MFMA at MI = 4, 5 at MI = 3) so they issue while this
// slice's MFMAs run.
template <int MI>
__device__ __forceinline__ void interleave_slice() {
  constexpr int kValu = (8 * (MI + 4) + 4 * MI - 1) / (4 * MI);
#pragma unroll
  for (int i = 0; i < 4 * MI; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
    __builtin_amdgcn_sched_group_barrier(0x002, kValu, 0);   // VALU
  }
}

// Slice KS of a step: MFMAs on `cur` while dequantizing slice KS+1 into `nxt`.
template <int KS, int MI>
__device__ __forceinline__ void pipelined_slice(floatx16 (&acc)[MI][4], const FragT<MI>& cur,
                                                FragT<MI>& nxt, const uint32_t (&a_raw)[MI][8],
                                                const uint32_t (&b_raw)[4][8],
                                                const uint2 (&a_sc)[MI], const uint2 (&b_sc)[4]) {
  if constexpr (KS + 1 < 8) dequant_slice<KS + 1>(nxt, a_raw, b_raw, a_sc, b_sc);
  mfma_slice(acc, cur);
  interleave_slice<MI>();
}

// LDS beyond the default 64 KiB is opted into once per kernel and device.
hipError_t launch_with_lds(void (*kernel)(Params), size_t lds, int grid, hipStream_t s,
                           const Params& p);

// Family launchers (one translation unit each).  `grid` = tiles_m * tiles_n.
hipError_t launch_two_level_0(bool fast, int scv, const Params& p, int grid, hipStream_t s);
hipError_t launch_two_level_1(bool fast, int scv, const Params& p, int grid, hipStream_t s);
// gemm_nv_dma.hip, one object per format (0 NVFP4, 1 UE5M3) and tile height
// (4: 256 rows, 3: 192 rows)
hipError_t launch_two_level_dma_0_4(int scv, const Params& p, hipStream_t s);
hipError_t launch_two_level_dma_0_3(int scv, const Params& p, hipStream_t s);
hipError_t launch_two_level_dma_1_4(int scv, const Params& p, hipStream_t s);
hipError_t launch_two_level_dma_1_3(int scv, const Params& p, hipStream_t s);
hipError_t launch_mx(bool fast, int scv, const Params& p, int grid, hipStream_t s);
hipError_t launch_mx_ring(const Params& p, int grid, hipStream_t s);
hipError_t launch_mx_tiled(const Params& p, int grid, hipStream_t s);

}  // namespace fp4gemm
