// Block-scaled FP4 GEMMs for gfx950 (NVFP4 pretraining paper, App. B.3:
// per-block partial products scaled by both local decode scales, fp32
// accumulation, the two global decode scales applied to the output; §4.1 /
// Fig. 5: Fprop, Dgrad and Wgrad all run this product on FP4 operands).
//
//   D[M, N] (+)= s_A s_B sum_k a[m, k] b[n, k],   a = e2m1 * scale ("TN")
//
// Every kernel uses one skeleton: a 256 x 256 output tile per workgroup,
// four waves in a 2 x 2 arrangement (128 x 128 each, 4 x 4 MFMA tiles of
// 32 x 32), FP4 codes and scales staged through LDS, one barrier per K step,
// the next K step's loads in flight while the current one is multiplied,
// and an XCD-aware grouped tile order.
//
// * NVFP4 / UE5M3: e2m1 * scale is exact in fp16 (E4M3 products lie in
//   [2^-10, 2688]; UE5M3 scales are pre-multiplied by 2^-5 so products lie
//   in [2^-23, 23040] on fp16's 2^-24 grid), so every lane dequantizes its
//   own MFMA fragment in registers -- a hardware FP4->fp16 convert and a
//   packed fp16 multiply by the block scale -- and feeds
//   v_mfma_f32_32x32x16_f16 with fp32 accumulation.  The 2^-5 shifts and
//   the tensor scales are applied to the fp32 result.
//     k_gemm_two_level_dma  NVFP4, K % 256 == 0, 16-byte code rows: codes
//                           go to LDS by DMA (global_load_lds).
//     k_gemm_two_level      every other shape (and UE5M3): codes staged
//                           through registers, ragged edges masked.
// * MXFP4: gfx950's scaled MFMA takes FP4 operands and one E8M0 scale per 32
//   K-values per lane, which is exactly an MXFP4 block, so the codes go from
//   LDS to v_mfma_scale_f32_32x32x64_f8f6f4 untouched.
//     k_gemm_mx_tiled  TILED scales, K % 512 == 0: K step 256, codes and
//                      scales by DMA in whole 128-byte lines.
//     k_gemm_mx_ring   K % 512 == 0, other scale layouts: 4-stage K-128 DMA ring.
//     k_gemm_mx        every other shape: register-staged, edges masked.
//
// The order of K inside one K step is free as long as A and B agree: lane
// half h of a wave owns a contiguous half of the step's K range for both
// operands, so each lane's codes are one contiguous run in LDS.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fp4_device.hpp"
#include "fp4_internal.hpp"

using namespace fp4dev;

namespace {

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
  float* D;
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
__device__ __forceinline__ void epilogue(const Params& p, floatx16 (&acc)[4][4], float scale,
                                         int64_t m0, int64_t n0, int wm, int wn, int lane) {
  const int i = lane & 31, h = lane >> 5;
  const bool vec = (p.ldd & 3) == 0 && (reinterpret_cast<uintptr_t>(p.D) & 15) == 0;
#pragma unroll
  for (int mi = 0; mi < 4; ++mi) {
    const int64_t row = m0 + wm * 128 + mi * 32 + i;
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

// ------------------------------------------------------- NVFP4 / UE5M3 --
constexpr int kBK2 = 128;   // K per step: 64 code bytes and 8 scales per row

// Two consecutive block scales (codes in bits 0-7 and 8-15) as an fp16
// pair, block 2k in the low half.  E4M3 uses the packed hardware FP8 -> fp16
// convert with a unit scale (exact: every E4M3 value, subnormals included,
// is an fp16 value); UE5M3 is decoded arithmetically and pre-multiplied by
// 2^-5 (exact).
template <int FMT>
__device__ __forceinline__ uint32_t scale_pair_f16(uint32_t two_codes) {
  if constexpr (FMT == kNV) {
    return __builtin_bit_cast(uint32_t,
                              __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(two_codes, 1.0f, false));
  } else {
    const _Float16 lo = static_cast<_Float16>(scale_m3_decode<15>(two_codes & 0xFFu) * 0x1p-5f);
    const _Float16 hi =
        static_cast<_Float16>(scale_m3_decode<15>((two_codes >> 8) & 0xFFu) * 0x1p-5f);
    return __builtin_bit_cast(uint32_t, half2v{lo, hi});
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
// 8 K-values of its row for each of the wave's 4 A and 4 B tiles.
struct Frag {
  half8 a[4], b[4];
};

template <int KS>
__device__ __forceinline__ void dequant_slice(Frag& f, const uint32_t (&a_raw)[4][8],
                                              const uint32_t (&b_raw)[4][8], const uint2 (&a_sc)[4],
                                              const uint2 (&b_sc)[4]) {
  constexpr int W = KS >> 1;     // block of the lane's 4: one 16-element block per two slices
#pragma unroll
  for (int mi = 0; mi < 4; ++mi)
    f.a[mi] = dequant8<W & 1>(a_raw[mi][KS], (W >> 1) ? a_sc[mi].y : a_sc[mi].x);
#pragma unroll
  for (int ni = 0; ni < 4; ++ni)
    f.b[ni] = dequant8<W & 1>(b_raw[ni][KS], (W >> 1) ? b_sc[ni].y : b_sc[ni].x);
}

__device__ __forceinline__ void mfma_slice(floatx16 (&acc)[4][4], const Frag& f) {
#pragma unroll
  for (int mi = 0; mi < 4; ++mi)
#pragma unroll
    for (int ni = 0; ni < 4; ++ni)
      acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_f16(f.b[ni], f.a[mi], acc[mi][ni], 0, 0, 0);
}

// Scheduling hint for one slice: alternate one MFMA with four VALU ops so
// the next slice's dequantization issues while this slice's MFMAs run.
__device__ __forceinline__ void interleave_slice() {
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
    __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);   // VALU
  }
}

// Slice KS of a step: MFMAs on `cur` while dequantizing slice KS+1 into `nxt`.
template <int KS>
__device__ __forceinline__ void pipelined_slice(floatx16 (&acc)[4][4], const Frag& cur, Frag& nxt,
                                                const uint32_t (&a_raw)[4][8],
                                                const uint32_t (&b_raw)[4][8],
                                                const uint2 (&a_sc)[4], const uint2 (&b_sc)[4]) {
  if constexpr (KS + 1 < 8) dequant_slice<KS + 1>(nxt, a_raw, b_raw, a_sc, b_sc);
  mfma_slice(acc, cur);
  interleave_slice();
}

template <int FMT, bool FAST, int SCV>
__global__ __launch_bounds__(kThreads, 1) void k_gemm_two_level(Params p) {
  extern __shared__ uint4 smem_raw[];
  Stage2* st = reinterpret_cast<Stage2*>(smem_raw);
  int tm, tn;
  tile_coords(p, tm, tn);
  const int64_t m0 = static_cast<int64_t>(tm) * kBM, n0 = static_cast<int64_t>(tn) * kBN;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t row_bytes = p.K >> 1;
  const int64_t kblocks = p.K >> 4;
  const int nsteps = static_cast<int>((p.K + kBK2 - 1) / kBK2);
  const int64_t lim[2] = {p.M, p.N};
  const int64_t base[2] = {m0, n0};

  // Staging registers for the next K step.  Loaded values are kept raw and
  // only masked/decoded when written to LDS, so no load has to be waited for
  // before the MFMAs of the current step are issued.
  uint4 rc[2][4];        // codes: 4 chunks per operand per thread
  uint2 rs[2];           // scale bytes of row t: the step's 8 K-blocks (packed)
  uint32_t rsb[2][8];    // the same as 8 separate bytes (strided scale rows)
  uint32_t valid[2];     // bit j: chunk j's row is inside the matrix; bit 4: row t is

  auto load_step = [&](int s) {
    const int64_t k0b = static_cast<int64_t>(s) * (kBK2 / 2);
    if constexpr (FAST) {
#pragma unroll
      for (int o = 0; o < 2; ++o) {
        const uint8_t* sp = scale_ptr(p, o, base[o] + t, static_cast<int64_t>(s) * 8);
        if ((SCV >> o) & 1) {
          rs[o] = *reinterpret_cast<const uint2*>(sp);
        } else {
          // 8 independent byte loads, used only when the scales are stored
          const int64_t st = p.s_kblk[o];
#pragma unroll
          for (int kb = 0; kb < 8; ++kb) rsb[o][kb] = sp[kb * st];
        }
        valid[o] = 31u;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int c = t + kThreads * j;
          rc[o][j] = *reinterpret_cast<const uint4*>(p.codes[o] + (base[o] + (c >> 2)) * p.ld[o] +
                                                     k0b + (c & 3) * 16);
        }
      }
      return;
    }
    const bool kfull = k0b + kBK2 / 2 <= row_bytes;
#pragma unroll
    for (int o = 0; o < 2; ++o) {
      // scales first: they are consumed first
      const int64_t gr = base[o] + t;
      const bool rv = gr < lim[o];
      const uint8_t* sp = scale_ptr(p, o, rv ? gr : lim[o] - 1, static_cast<int64_t>(s) * 8);
      if (kfull && p.sc_vec[o]) {
        rs[o] = *reinterpret_cast<const uint2*>(sp);
      } else {
        uint32_t lo = 0, hi = 0;
#pragma unroll
        for (int kb = 0; kb < 8; ++kb) {
          const uint32_t v =
              (static_cast<int64_t>(s) * 8 + kb < kblocks) ? sp[kb * p.s_kblk[o]] : 0u;
          if (kb < 4) lo |= v << (8 * kb);
          else hi |= v << (8 * (kb - 4));
        }
        rs[o] = make_uint2(lo, hi);
      }
      uint32_t vb = rv ? 16u : 0u;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int c = t + kThreads * j;
        const int64_t r = base[o] + (c >> 2);
        vb |= (r < lim[o] ? 1u : 0u) << j;
      }
      valid[o] = vb;
      if (kfull && p.vec16[o]) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int c = t + kThreads * j;
          const int64_t r = base[o] + (c >> 2);
          const uint8_t* src = p.codes[o] + (r < lim[o] ? r : lim[o] - 1) * p.ld[o];
          rc[o][j] = *reinterpret_cast<const uint4*>(src + k0b + (c & 3) * 16);
        }
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int c = t + kThreads * j;
          const int64_t r = base[o] + (c >> 2);
          const uint8_t* src = p.codes[o] + (r < lim[o] ? r : lim[o] - 1) * p.ld[o];
          rc[o][j] = load_codes16(src, k0b + (c & 3) * 16, row_bytes, p.vec16[o]);
        }
      }
    }
  };
  auto store_scales = [&](Stage2& S) {
#pragma unroll
    for (int o = 0; o < 2; ++o) {
      const bool rv = valid[o] & 16u;
      const bool bytes = FAST && !((SCV >> o) & 1);
      // fp16 pairs of the step's 8 scale codes (pair k: blocks 2k, 2k + 1);
      // strided scales arrive as separate bytes, each pair needs only its two
      uint32_t pr[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const uint32_t two = bytes ? rsb[o][2 * k] | (rsb[o][2 * k + 1] << 8)
                                   : (k < 2 ? rs[o].x : rs[o].y) >> (16 * (k & 1));
        pr[k] = scale_pair_f16<FMT>(two);
      }
      S.scales[o][0][t] = rv ? make_uint2(pr[0], pr[1]) : make_uint2(0u, 0u);
      S.scales[o][1][t] = rv ? make_uint2(pr[2], pr[3]) : make_uint2(0u, 0u);
    }
  };
  auto store_codes = [&](Stage2& S) {
#pragma unroll
    for (int o = 0; o < 2; ++o) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int c = t + kThreads * j;
        const int row = c >> 2, q = c & 3;
        S.codes[o][q][row ^ (q << 2)] = (valid[o] >> j) & 1u ? rc[o][j] : make_uint4(0u, 0u, 0u, 0u);
      }
    }
  };

  floatx16 acc[4][4];
#pragma unroll
  for (int mi = 0; mi < 4; ++mi)
#pragma unroll
    for (int ni = 0; ni < 4; ++ni) acc[mi][ni] = floatx16{};

  const int i = lane & 31, h = lane >> 5;
  uint32_t a_raw[4][8], b_raw[4][8];
  uint2 a_sc[4], b_sc[4];
  // this lane's raw codes (its K half of the step) and decoded scales
  auto read_stage = [&](const Stage2& S) {
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) {
      const int row = wm * 128 + mi * 32 + i;
      const uint4 c0 = S.codes[0][2 * h][row ^ ((2 * h) << 2)];
      const uint4 c1 = S.codes[0][2 * h + 1][row ^ ((2 * h + 1) << 2)];
      a_raw[mi][0] = c0.x; a_raw[mi][1] = c0.y; a_raw[mi][2] = c0.z; a_raw[mi][3] = c0.w;
      a_raw[mi][4] = c1.x; a_raw[mi][5] = c1.y; a_raw[mi][6] = c1.z; a_raw[mi][7] = c1.w;
      a_sc[mi] = S.scales[0][h][row];
    }
#pragma unroll
    for (int ni = 0; ni < 4; ++ni) {
      const int row = wn * 128 + ni * 32 + i;
      const uint4 c0 = S.codes[1][2 * h][row ^ ((2 * h) << 2)];
      const uint4 c1 = S.codes[1][2 * h + 1][row ^ ((2 * h + 1) << 2)];
      b_raw[ni][0] = c0.x; b_raw[ni][1] = c0.y; b_raw[ni][2] = c0.z; b_raw[ni][3] = c0.w;
      b_raw[ni][4] = c1.x; b_raw[ni][5] = c1.y; b_raw[ni][6] = c1.z; b_raw[ni][7] = c1.w;
      b_sc[ni] = S.scales[1][h][row];
    }
  };
  if (nsteps > 0) {
    load_step(0);
    store_scales(st[0]);
    store_codes(st[0]);
    __syncthreads();
    read_stage(st[0]);
  }
  // Step s: the raw codes and scales of stage s & 1 are already in
  // registers.  The next step's stage is loaded and stored during slices
  // 0..5; its raw registers are dead once slice 7 has been dequantized
  // (during slice 6), so the barrier comes before slice 7 and the next
  // stage's LDS reads overlap slice 7's MFMAs instead of stalling the top of
  // the next step.  The stage written during step s + 1 (= s & 1) was last
  // read before this barrier.  Every step loads and stores a next step (the
  // last one re-reads itself into the buffer nobody reads again): with no
  // branch around them the loads and LDS writes share one scheduling region
  // with the MFMAs.
  for (int s = 0; s < nsteps; ++s) {
    load_step(s + 1 < nsteps ? s + 1 : s);
    Frag f0, f1;
    dequant_slice<0>(f0, a_raw, b_raw, a_sc, b_sc);
    pipelined_slice<0>(acc, f0, f1, a_raw, b_raw, a_sc, b_sc);
    pipelined_slice<1>(acc, f1, f0, a_raw, b_raw, a_sc, b_sc);
    pipelined_slice<2>(acc, f0, f1, a_raw, b_raw, a_sc, b_sc);
    pipelined_slice<3>(acc, f1, f0, a_raw, b_raw, a_sc, b_sc);
    store_scales(st[(s + 1) & 1]);
    pipelined_slice<4>(acc, f0, f1, a_raw, b_raw, a_sc, b_sc);
    pipelined_slice<5>(acc, f1, f0, a_raw, b_raw, a_sc, b_sc);
    store_codes(st[(s + 1) & 1]);
    pipelined_slice<6>(acc, f0, f1, a_raw, b_raw, a_sc, b_sc);
    __syncthreads();
    read_stage(st[(s + 1) & 1]);
    pipelined_slice<7>(acc, f1, f0, a_raw, b_raw, a_sc, b_sc);
  }

  float scale = FMT == kUE ? 1024.0f : 1.0f;   // undo the two 2^-5 scale shifts
  if (p.s_dec[0]) scale *= *p.s_dec[0];
  // s_B is applied as a second multiply so that s_A * s_B never under/overflows alone
  const float sb = p.s_dec[1] ? *p.s_dec[1] : 1.0f;
#pragma unroll
  for (int mi = 0; mi < 4; ++mi)
#pragma unroll
    for (int ni = 0; ni < 4; ++ni) acc[mi][ni] *= scale;
  epilogue(p, acc, sb, m0, n0, wm, wn, lane);
}

// -------------------------------------------------------------- MXFP4 ---
constexpr int kBKX = 128;   // K per step: 64 code bytes and 4 E8M0 scales per row

struct StageX {
  // codes: [operand][chunk q 0..3][row slot][16 B], slot = row ^ (q << 2)
  uint4 codes[2][4][256];
  // scales: [operand][row] -> the 4 E8M0 bytes of the step's blocks
  uint32_t scales[2][256];
};

// One 64-K slice: lane half h owns the 32 K-values of chunk 2h + KS (one
// MXFP4 block); its E8M0 scale is byte KS of the lane's (pre-shifted) word.
template <int KS>
__device__ __forceinline__ void mx_slice(const StageX& S, floatx16 (&acc)[4][4],
                                         const uint32_t (&a_sc)[4], const uint32_t (&b_sc)[4],
                                         int wm, int wn, int i, int h) {
  const int q = 2 * h + KS;
  int8v a_op[4], b_op[4];
#pragma unroll
  for (int mi = 0; mi < 4; ++mi) {
    const int row = wm * 128 + mi * 32 + i;
    const uint4 c = S.codes[0][q][row ^ (q << 2)];
    a_op[mi] = int8v{(int)c.x, (int)c.y, (int)c.z, (int)c.w, 0, 0, 0, 0};
  }
#pragma unroll
  for (int ni = 0; ni < 4; ++ni) {
    const int row = wn * 128 + ni * 32 + i;
    const uint4 c = S.codes[1][q][row ^ (q << 2)];
    b_op[ni] = int8v{(int)c.x, (int)c.y, (int)c.z, (int)c.w, 0, 0, 0, 0};
  }
#pragma unroll
  for (int mi = 0; mi < 4; ++mi)
#pragma unroll
    for (int ni = 0; ni < 4; ++ni)
      acc[mi][ni] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
          b_op[ni], a_op[mi], acc[mi][ni], 4, 4, KS, static_cast<int>(b_sc[ni]), KS,
          static_cast<int>(a_sc[mi]));
}

template <bool FAST, int SCV>
__global__ __launch_bounds__(kThreads, 1) void k_gemm_mx(Params p) {
  extern __shared__ uint4 smem_raw[];
  StageX* st = reinterpret_cast<StageX*>(smem_raw);
  int tm, tn;
  tile_coords(p, tm, tn);
  const int64_t m0 = static_cast<int64_t>(tm) * kBM, n0 = static_cast<int64_t>(tn) * kBN;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t kblocks = p.K >> 5;
  const int nsteps = static_cast<int>((p.K + kBKX - 1) / kBKX);
  const int64_t lim[2] = {p.M, p.N};
  const int64_t base[2] = {m0, n0};

  uint4 rc[2][4];        // staged codes: 4 chunks (one MXFP4 block each) per operand
  uint32_t rs[2];        // E8M0 scales of row t for the step's 4 blocks
  uint32_t valid[2];     // bit j: chunk j's row is inside the matrix; bit 4: row t is

  auto load_step = [&](int s) {
    const int64_t k0b = static_cast<int64_t>(s) * (kBKX / 2);
    if constexpr (FAST) {
#pragma unroll
      for (int o = 0; o < 2; ++o) {
        const uint8_t* sp = scale_ptr(p, o, base[o] + t, static_cast<int64_t>(s) * 4);
        if ((SCV >> o) & 1) {
          rs[o] = *reinterpret_cast<const uint32_t*>(sp);
        } else {
          const int64_t st = p.s_kblk[o];
          rs[o] = sp[0] | (sp[st] << 8) | (sp[2 * st] << 16) | (sp[3 * st] << 24);
        }
        valid[o] = 31u;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int c = t + kThreads * j;
          rc[o][j] = *reinterpret_cast<const uint4*>(p.codes[o] + (base[o] + (c >> 2)) * p.ld[o] +
                                                     k0b + (c & 3) * 16);
        }
      }
      return;
    }
    const bool kfull = (static_cast<int64_t>(s) + 1) * 4 <= kblocks;
#pragma unroll
    for (int o = 0; o < 2; ++o) {
      const int64_t gr = base[o] + t;
      const bool rv = gr < lim[o];
      const uint8_t* sp = scale_ptr(p, o, rv ? gr : lim[o] - 1, static_cast<int64_t>(s) * 4);
      if (kfull && p.sc_vec[o]) {
        rs[o] = *reinterpret_cast<const uint32_t*>(sp);
      } else {
        uint32_t w = 0;
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
          if (static_cast<int64_t>(s) * 4 + kb < kblocks)
            w |= static_cast<uint32_t>(sp[kb * p.s_kblk[o]]) << (8 * kb);
        rs[o] = w;
      }
      uint32_t vb = rv ? 16u : 0u;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int c = t + kThreads * j;
        const int64_t r = base[o] + (c >> 2);
        vb |= (r < lim[o] ? 1u : 0u) << j;
      }
      valid[o] = vb;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int c = t + kThreads * j;
        const int64_t r = base[o] + (c >> 2);
        const int q = c & 3;
        const uint8_t* src = p.codes[o] + (r < lim[o] ? r : lim[o] - 1) * p.ld[o] + k0b + q * 16;
        // K % 32 == 0: a 16-byte chunk is one whole MXFP4 block or absent
        if (kfull) rc[o][j] = *reinterpret_cast<const uint4*>(src);
        else rc[o][j] = (static_cast<int64_t>(s) * 4 + q < kblocks)
                            ? *reinterpret_cast<const uint4*>(src) : make_uint4(0u, 0u, 0u, 0u);
      }
    }
  };
  auto store_step = [&](StageX& S) {
#pragma unroll
    for (int o = 0; o < 2; ++o) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int c = t + kThreads * j;
        const int row = c >> 2, q = c & 3;
        S.codes[o][q][row ^ (q << 2)] = (valid[o] >> j) & 1u ? rc[o][j] : make_uint4(0u, 0u, 0u, 0u);
      }
      S.scales[o][t] = (valid[o] & 16u) ? rs[o] : 0u;
    }
  };

  floatx16 acc[4][4];
#pragma unroll
  for (int mi = 0; mi < 4; ++mi)
#pragma unroll
    for (int ni = 0; ni < 4; ++ni) acc[mi][ni] = floatx16{};

  const int i = lane & 31, h = lane >> 5;
  if (nsteps > 0) {
    load_step(0);
    store_step(st[0]);
    __syncthreads();
  }
  for (int s = 0; s < nsteps; ++s) {
    const bool more = s + 1 < nsteps;
    if (more) load_step(s + 1);
    const StageX& S = st[s & 1];
    // lane half h uses blocks 2h and 2h+1: shift them down to bytes 0 and 1
    uint32_t a_sc[4], b_sc[4];
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) a_sc[mi] = S.scales[0][wm * 128 + mi * 32 + i] >> (16 * h);
#pragma unroll
    for (int ni = 0; ni < 4; ++ni) b_sc[ni] = S.scales[1][wn * 128 + ni * 32 + i] >> (16 * h);
    mx_slice<0>(S, acc, a_sc, b_sc, wm, wn, i, h);
    mx_slice<1>(S, acc, a_sc, b_sc, wm, wn, i, h);
    if (more) store_step(st[(s + 1) & 1]);
    __syncthreads();
  }
  epilogue(p, acc, 1.0f, m0, n0, wm, wn, lane);
}

// ------------------------------------------------- MXFP4, LDS-DMA ring ---
// The same product for the common case (K a multiple of 128, contiguous
// 4-byte-aligned scale rows): codes and scales go from global memory
// straight into LDS (gfx950 global_load_lds, 16- and 4-byte forms) through
// a ring of four K-step stages, so no registers hold staged data and three
// K steps of loads are in flight behind the MFMAs.  Out-of-range rows of a
// ragged M or N read the last valid row; their outputs are never stored.
//
// Each stage sits in its own __shared__ variable and is named with a
// compile-time index, so the compiler can tell the stages apart and does not
// drain every outstanding DMA before each LDS read; the waits for the DMA
// are the explicit vmcnt waits below, one barrier per K step.
constexpr int kStagesX = 4;
constexpr int kDmaPerStep = 10;   // per wave: 2 x 4 code chunks + 2 scale rows

struct StageD {
  uint4 codes[2][1024];     // [operand][row * 4 + (chunk ^ dma_swizzle(row))]
  uint32_t scales[2][256];  // [operand][row]: E8M0 bytes of the step's 4 blocks
};

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

struct DmaSrc {
  const uint8_t* codes[2][4];   // this lane's chunk of rows wave*64 + 16j + lane/4
  const uint8_t* scales[2];     // scales of K step 0 of this lane's row wave*64 + lane
  int tiled[2];
};

__device__ __forceinline__ void dma_step(StageD& S, const DmaSrc& src, int64_t step, int wave) {
  const int64_t cb = step * (kBKX / 2);
#pragma unroll
  for (int o = 0; o < 2; ++o)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      __builtin_amdgcn_global_load_lds(src.codes[o][j] + cb, &S.codes[o][wave * 256 + j * 64], 16, 0, 0);
  // the 4 scale bytes of K step `step`: row-major at 4 step, TILED in atom
  // step / 2 at byte 4 (step % 2) of the row's 8
#pragma unroll
  for (int o = 0; o < 2; ++o) {
    const int64_t sb = src.tiled[o] ? ((step >> 1) << 11) + ((step & 1) << 2) : step * 4;
    __builtin_amdgcn_global_load_lds(src.scales[o] + sb, &S.scales[o][wave * 64], 4, 0, 0);
  }
}

struct MxFrag {
  int8v a[4], b[4];
};

template <int KS>
__device__ __forceinline__ void ring_operands(const StageD& S, MxFrag& f, int wm, int wn, int i,
                                              int h) {
  const int q = 2 * h + KS;
#pragma unroll
  for (int mi = 0; mi < 4; ++mi) {
    const int row = wm * 128 + mi * 32 + i;
    const uint4 c = S.codes[0][row * 4 + (q ^ dma_swizzle(row))];
    f.a[mi] = int8v{(int)c.x, (int)c.y, (int)c.z, (int)c.w, 0, 0, 0, 0};
  }
#pragma unroll
  for (int ni = 0; ni < 4; ++ni) {
    const int row = wn * 128 + ni * 32 + i;
    const uint4 c = S.codes[1][row * 4 + (q ^ dma_swizzle(row))];
    f.b[ni] = int8v{(int)c.x, (int)c.y, (int)c.z, (int)c.w, 0, 0, 0, 0};
  }
}

__device__ __forceinline__ void ring_scales(const StageD& S, uint32_t (&a_sc)[4],
                                            uint32_t (&b_sc)[4], int wm, int wn, int i, int h) {
#pragma unroll
  for (int mi = 0; mi < 4; ++mi) a_sc[mi] = S.scales[0][wm * 128 + mi * 32 + i] >> (16 * h);
#pragma unroll
  for (int ni = 0; ni < 4; ++ni) b_sc[ni] = S.scales[1][wn * 128 + ni * 32 + i] >> (16 * h);
}

template <int KS>
__device__ __forceinline__ void ring_mfma(floatx16 (&acc)[4][4], const MxFrag& f,
                                          const uint32_t (&a_sc)[4], const uint32_t (&b_sc)[4]) {
#pragma unroll
  for (int mi = 0; mi < 4; ++mi)
#pragma unroll
    for (int ni = 0; ni < 4; ++ni)
      acc[mi][ni] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
          f.b[ni], f.a[mi], acc[mi][ni], 4, 4, KS, static_cast<int>(b_sc[ni]), KS,
          static_cast<int>(a_sc[mi]));
}

// One K step on stage C whose slice-0 operands f0 and scales are already in
// registers.  Slice 1 is read and slice 0 multiplied; then (unless this is
// the last step) the barrier at which the next stage Nx has landed for every
// wave (at most WAIT of this wave's DMA still in flight) and C is no longer
// read by anyone, so C is refilled with K step `refill` (if DMA) while slice
// 1 is multiplied and Nx's slice 0 and scales are read.
template <bool LAST, bool DMA, int WAIT>
__device__ __forceinline__ void ring_step(StageD& C, const StageD& Nx, floatx16 (&acc)[4][4],
                                          MxFrag& f0, MxFrag& f1, uint32_t (&a_sc)[4],
                                          uint32_t (&b_sc)[4], const DmaSrc& src, int refill,
                                          int wave, int wm, int wn, int i, int h) {
  ring_operands<1>(C, f1, wm, wn, i, h);
  ring_mfma<0>(acc, f0, a_sc, b_sc);
  if constexpr (LAST) {
    ring_mfma<1>(acc, f1, a_sc, b_sc);
  } else {
    wait_vmcnt<WAIT>();
    ring_barrier();
    if constexpr (DMA) dma_step(C, src, refill, wave);
    uint32_t na[4], nb[4];
    ring_scales(Nx, na, nb, wm, wn, i, h);
    ring_operands<0>(Nx, f0, wm, wn, i, h);
    ring_mfma<1>(acc, f1, a_sc, b_sc);
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      a_sc[x] = na[x];
      b_sc[x] = nb[x];
    }
  }
}

// K is a multiple of 4 K steps (512), so the ring turns whole: every step
// of the main loop refills the stage it has just finished (10 DMA per wave
// per step, so waiting for the next stage leaves 2 steps = 20 in flight),
// and the last four steps drain it with compile-time waits.
__global__ __launch_bounds__(kThreads, 1) void k_gemm_mx_ring(Params p) {
  __shared__ StageD st0, st1, st2, st3;
  int tm, tn;
  tile_coords(p, tm, tn);
  const int64_t m0 = static_cast<int64_t>(tm) * kBM, n0 = static_cast<int64_t>(tn) * kBN;
  const int t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int nsteps = static_cast<int>(p.K / kBKX);
  const int64_t lim[2] = {p.M, p.N};
  const int64_t base[2] = {m0, n0};

  DmaSrc src;
#pragma unroll
  for (int o = 0; o < 2; ++o) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int row = wave * 64 + j * 16 + (lane >> 2);
      const int q = (lane & 3) ^ dma_swizzle(row);
      const int64_t r = min(base[o] + row, lim[o] - 1);
      src.codes[o][j] = p.codes[o] + r * p.ld[o] + q * 16;
    }
    const int64_t r = min(base[o] + wave * 64 + lane, lim[o] - 1);
    src.scales[o] = scale_ptr(p, o, r, 0);
    src.tiled[o] = p.tiled[o];
  }

  floatx16 acc[4][4];
#pragma unroll
  for (int mi = 0; mi < 4; ++mi)
#pragma unroll
    for (int ni = 0; ni < 4; ++ni) acc[mi][ni] = floatx16{};

  const int i = lane & 31, h = lane >> 5;
  dma_step(st0, src, 0, wave);
  dma_step(st1, src, 1, wave);
  dma_step(st2, src, 2, wave);
  dma_step(st3, src, 3, wave);
  wait_vmcnt<3 * kDmaPerStep>();
  ring_barrier();
  MxFrag f0, f1;
  uint32_t a_sc[4], b_sc[4];
  ring_scales(st0, a_sc, b_sc, wm, wn, i, h);
  ring_operands<0>(st0, f0, wm, wn, i, h);
  constexpr int W2 = 2 * kDmaPerStep;
  for (int k = 0; k + 4 < nsteps; k += 4) {
    ring_step<false, true, W2>(st0, st1, acc, f0, f1, a_sc, b_sc, src, k + 4, wave, wm, wn, i, h);
    ring_step<false, true, W2>(st1, st2, acc, f0, f1, a_sc, b_sc, src, k + 5, wave, wm, wn, i, h);
    ring_step<false, true, W2>(st2, st3, acc, f0, f1, a_sc, b_sc, src, k + 6, wave, wm, wn, i, h);
    ring_step<false, true, W2>(st3, st0, acc, f0, f1, a_sc, b_sc, src, k + 7, wave, wm, wn, i, h);
  }
  ring_step<false, false, W2>(st0, st1, acc, f0, f1, a_sc, b_sc, src, 0, wave, wm, wn, i, h);
  ring_step<false, false, kDmaPerStep>(st1, st2, acc, f0, f1, a_sc, b_sc, src, 0, wave, wm, wn, i, h);
  ring_step<false, false, 0>(st2, st3, acc, f0, f1, a_sc, b_sc, src, 0, wave, wm, wn, i, h);
  ring_step<true, false, 0>(st3, st0, acc, f0, f1, a_sc, b_sc, src, 0, wave, wm, wn, i, h);
  epilogue(p, acc, 1.0f, m0, n0, wm, wn, lane);
}

// --------------------------------------- MXFP4, TILED scales, K step 256 ---
// With both operands' scales in the TILED layout and K a multiple of 512,
// one K step is 256: each code row contributes one full 128-byte line and
// the tile's scales one 2 KiB atom per operand, so the DMA reads whole lines
// only (16 per 16-byte DMA instruction of 8 rows, 16 per scale atom) instead
// of half lines and scattered 4-byte pieces.  Two stages of 68 KiB ping-pong;
// the barrier sits three quarters into each step, where the next stage has
// landed and the current one has been read, so the refill of the current
// stage overlaps the last quarter and the whole next step.
constexpr int kBKV = 256;
constexpr int kDmaV = 17;         // per wave and step: 2 x 8 code instructions + 1 scale

struct StageV {
  uint4 codes[2][2048];     // [operand][row * 8 + (chunk ^ v_swizzle(row))]
  uint2 scales[2][256];     // [operand][row]: E8M0 bytes of the step's 8 blocks
};

// Chunk q (0..7) of LDS row r sits at position q ^ v_swizzle(r): 8
// consecutive rows reading the same chunk use 8 distinct 16-byte bank
// groups, and so do the 8 rows of each parity among 16 consecutive rows.
__device__ __forceinline__ int v_swizzle(int row) { return (row & 7) ^ ((row >> 3) & 1); }

struct DmaSrcV {
  const uint8_t* codes[2][8];   // this lane's 16 bytes of rows wave*64 + 8j + lane/8
  const uint8_t* scales;        // this wave's half (wave & 1) of operand (wave >> 1)'s atom
};

__device__ __forceinline__ void dma_v(StageV& S, const DmaSrcV& src, int64_t step, int wave) {
  const int64_t cb = step * (kBKV / 2);
#pragma unroll
  for (int o = 0; o < 2; ++o)
#pragma unroll
    for (int j = 0; j < 8; ++j)
      __builtin_amdgcn_global_load_lds(src.codes[o][j] + cb, &S.codes[o][wave * 512 + j * 64], 16,
                                       0, 0);
  // atoms of one 256-row band are consecutive, 2 KiB apart, one per step
  __builtin_amdgcn_global_load_lds(src.scales + (step << 11),
                                   &S.scales[wave >> 1][(wave & 1) * 128], 16, 0, 0);
}

// Lane half h takes the 32 K-values of chunk 4h + KS (one MXFP4 block) in
// slice KS; its E8M0 scale is byte KS of word h of the row's 8 scale bytes.
template <int KS>
__device__ __forceinline__ void v_operands(const StageV& S, MxFrag& f, int wm, int wn, int i,
                                           int h) {
  const int q = 4 * h + KS;
#pragma unroll
  for (int mi = 0; mi < 4; ++mi) {
    const int row = wm * 128 + mi * 32 + i;
    const uint4 c = S.codes[0][row * 8 + (q ^ v_swizzle(row))];
    f.a[mi] = int8v{(int)c.x, (int)c.y, (int)c.z, (int)c.w, 0, 0, 0, 0};
  }
#pragma unroll
  for (int ni = 0; ni < 4; ++ni) {
    const int row = wn * 128 + ni * 32 + i;
    const uint4 c = S.codes[1][row * 8 + (q ^ v_swizzle(row))];
    f.b[ni] = int8v{(int)c.x, (int)c.y, (int)c.z, (int)c.w, 0, 0, 0, 0};
  }
}

__device__ __forceinline__ void v_scales(const StageV& S, uint32_t (&a_sc)[4], uint32_t (&b_sc)[4],
                                         int wm, int wn, int i, int h) {
  const uint32_t* sa = reinterpret_cast<const uint32_t*>(S.scales[0]);
  const uint32_t* sb = reinterpret_cast<const uint32_t*>(S.scales[1]);
#pragma unroll
  for (int mi = 0; mi < 4; ++mi) a_sc[mi] = sa[(wm * 128 + mi * 32 + i) * 2 + h];
#pragma unroll
  for (int ni = 0; ni < 4; ++ni) b_sc[ni] = sb[(wn * 128 + ni * 32 + i) * 2 + h];
}

// Slice 3 of a step with the refill of stage C (K step `refill`) woven in:
// one 16-byte code DMA after each of the 16 MFMAs, then the scale atom.
// Issued in one burst, the 68 DMA instructions of the workgroup would queue
// behind each other in the memory pipeline and hold back the MFMAs of every
// wave; left to the scheduler, they sink to the next barrier and do not
// overlap at all.  sched_barrier(0) pins each pair in place.
__device__ __forceinline__ void ring_mfma3_refill(floatx16 (&acc)[4][4], const MxFrag& f,
                                                  const uint32_t (&a_sc)[4],
                                                  const uint32_t (&b_sc)[4], StageV& C,
                                                  const DmaSrcV& src, int refill, int wave) {
  const int64_t cb = static_cast<int64_t>(refill) * (kBKV / 2);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int mi = 0; mi < 4; ++mi)
#pragma unroll
    for (int ni = 0; ni < 4; ++ni) {
      acc[mi][ni] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
          f.b[ni], f.a[mi], acc[mi][ni], 4, 4, 3, static_cast<int>(b_sc[ni]), 3,
          static_cast<int>(a_sc[mi]));
      const int x = mi * 4 + ni, o = x >> 3, j = x & 7;
      __builtin_amdgcn_global_load_lds(src.codes[o][j] + cb, &C.codes[o][wave * 512 + j * 64], 16,
                                       0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
  __builtin_amdgcn_global_load_lds(src.scales + (static_cast<int64_t>(refill) << 11),
                                   &C.scales[wave >> 1][(wave & 1) * 128], 16, 0, 0);
  __builtin_amdgcn_sched_barrier(0);
}

// One K step on stage C, slice-0 operands (fa) and scales in registers.
template <bool LAST, bool DMA>
__device__ __forceinline__ void v_step(StageV& C, const StageV& Nx, floatx16 (&acc)[4][4],
                                       MxFrag& fa, MxFrag& fb, uint32_t (&a_sc)[4],
                                       uint32_t (&b_sc)[4], const DmaSrcV& src, int refill,
                                       int wave, int wm, int wn, int i, int h) {
  v_operands<1>(C, fb, wm, wn, i, h);
  ring_mfma<0>(acc, fa, a_sc, b_sc);
  v_operands<2>(C, fa, wm, wn, i, h);
  ring_mfma<1>(acc, fb, a_sc, b_sc);
  v_operands<3>(C, fb, wm, wn, i, h);
  ring_mfma<2>(acc, fa, a_sc, b_sc);
  if constexpr (LAST) {
    ring_mfma<3>(acc, fb, a_sc, b_sc);
  } else {
    wait_vmcnt<0>();          // this wave's DMA of Nx (the only one in flight)
    ring_barrier();           // ... and every other wave's; C fully read
    uint32_t na[4], nb[4];
    v_scales(Nx, na, nb, wm, wn, i, h);
    v_operands<0>(Nx, fa, wm, wn, i, h);
    if constexpr (DMA) ring_mfma3_refill(acc, fb, a_sc, b_sc, C, src, refill, wave);
    else ring_mfma<3>(acc, fb, a_sc, b_sc);
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      a_sc[x] = na[x];
      b_sc[x] = nb[x];
    }
  }
}

__global__ __launch_bounds__(kThreads, 1) void k_gemm_mx_tiled(Params p) {
  __shared__ StageV sv0, sv1;
  int tm, tn;
  tile_coords(p, tm, tn);
  const int64_t m0 = static_cast<int64_t>(tm) * kBM, n0 = static_cast<int64_t>(tn) * kBN;
  const int t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int nsteps = static_cast<int>(p.K / kBKV);
  const int64_t lim[2] = {p.M, p.N};
  const int64_t base[2] = {m0, n0};

  DmaSrcV src;
#pragma unroll
  for (int o = 0; o < 2; ++o) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int row = wave * 64 + j * 8 + (lane >> 3);
      const int q = (lane & 7) ^ v_swizzle(row);
      const int64_t r = min(base[o] + row, lim[o] - 1);
      src.codes[o][j] = p.codes[o] + r * p.ld[o] + q * 16;
    }
  }
  {
    const int o = wave >> 1;
    src.scales = p.scales[o] + tiled_scale_offset(base[o], 0, p.kg) + (wave & 1) * 1024 + lane * 16;
  }

  floatx16 acc[4][4];
#pragma unroll
  for (int mi = 0; mi < 4; ++mi)
#pragma unroll
    for (int ni = 0; ni < 4; ++ni) acc[mi][ni] = floatx16{};

  const int i = lane & 31, h = lane >> 5;
  dma_v(sv0, src, 0, wave);
  dma_v(sv1, src, 1, wave);
  wait_vmcnt<kDmaV>();
  ring_barrier();
  MxFrag fa, fb;
  uint32_t a_sc[4], b_sc[4];
  v_scales(sv0, a_sc, b_sc, wm, wn, i, h);
  v_operands<0>(sv0, fa, wm, wn, i, h);
  for (int k = 0; k + 2 < nsteps; k += 2) {
    v_step<false, true>(sv0, sv1, acc, fa, fb, a_sc, b_sc, src, k + 2, wave, wm, wn, i, h);
    v_step<false, true>(sv1, sv0, acc, fa, fb, a_sc, b_sc, src, k + 3, wave, wm, wn, i, h);
  }
  v_step<false, false>(sv0, sv1, acc, fa, fb, a_sc, b_sc, src, 0, wave, wm, wn, i, h);
  v_step<true, false>(sv1, sv0, acc, fa, fb, a_sc, b_sc, src, 0, wave, wm, wn, i, h);
  epilogue(p, acc, 1.0f, m0, n0, wm, wn, lane);
}

// ------------------------------------------- NVFP4 / UE5M3, codes by DMA ---
// The two-level product for K a multiple of 256 and 16-byte-aligned code
// rows: the same per-lane dequantization and slice pipeline as
// k_gemm_two_level, but the codes go from global memory straight into LDS
// (global_load_lds, 16 bytes per lane) instead of through registers and LDS
// stores, and ragged M / N read the last valid row (never stored).  Block
// scales are still loaded to registers and decoded once per K step by the
// loading thread.  Codes and scales of each of the two stages are separate
// __shared__ variables named with compile-time indices, so the compiler can
// tell the DMA targets from the LDS the waves read and write.
constexpr int kDmaNv = 8;    // per wave and K step: 2 operands x 4 code instructions

struct DmaSrcNv {
  const uint8_t* base[2];       // operand code matrices (uniform)
  uint32_t off[2][4];           // this lane's 16 bytes of rows wave*64 + 16j + lane/4
};                              // (the host keeps every offset below 2^31)

__device__ __forceinline__ void dma_codes_nv(uint4 (&dst)[2][1024], const DmaSrcNv& src,
                                             int64_t step, int wave) {
  const int64_t cb = step * (kBK2 / 2);
#pragma unroll
  for (int o = 0; o < 2; ++o)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      __builtin_amdgcn_global_load_lds(src.base[o] + cb + src.off[o][j],
                                       &dst[o][wave * 256 + j * 64], 16, 0, 0);
}

template <int FMT, int SCV>
__global__ __launch_bounds__(kThreads, 1) void k_gemm_two_level_dma(Params p) {
  __shared__ uint4 cst0[2][1024], cst1[2][1024];   // [operand][row * 4 + (chunk ^ swizzle)]
  __shared__ uint2 sst0[2][2][256], sst1[2][2][256];  // [operand][half][row] fp16 scale pairs
  int tm, tn;
  tile_coords(p, tm, tn);
  const int64_t m0 = static_cast<int64_t>(tm) * kBM, n0 = static_cast<int64_t>(tn) * kBN;
  const int t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int nsteps = static_cast<int>(p.K / kBK2);
  const int64_t lim[2] = {p.M, p.N};
  const int64_t base[2] = {m0, n0};

  DmaSrcNv src;
#pragma unroll
  for (int o = 0; o < 2; ++o) {
    src.base[o] = p.codes[o];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int row = wave * 64 + j * 16 + (lane >> 2);
      const int q = (lane & 3) ^ dma_swizzle(row);
      const int64_t r = min(base[o] + row, lim[o] - 1);
      src.off[o][j] = static_cast<uint32_t>(r * p.ld[o] + q * 16);
    }
  }
  // scales of row t (clamped), K step s: a per-lane offset plus a uniform
  // per-step stride (one 2 KiB atom TILED, 8 K-blocks otherwise)
  uint32_t soff[2];
  int64_t sstep[2];
#pragma unroll
  for (int o = 0; o < 2; ++o) {
    soff[o] = static_cast<uint32_t>(scale_ptr(p, o, min(base[o] + t, lim[o] - 1), 0) - p.scales[o]);
    sstep[o] = p.tiled[o] ? 2048 : 8 * p.s_kblk[o];
  }

  uint2 rs[2];
  uint32_t rsb[2][8];
  auto load_scales = [&](int s) {
#pragma unroll
    for (int o = 0; o < 2; ++o) {
      const uint8_t* sp = p.scales[o] + s * sstep[o] + soff[o];
      if ((SCV >> o) & 1) {
        rs[o] = *reinterpret_cast<const uint2*>(sp);
      } else {
        const int64_t st = p.s_kblk[o];
#pragma unroll
        for (int kb = 0; kb < 8; ++kb) rsb[o][kb] = sp[kb * st];
      }
    }
  };
  auto store_scales = [&](uint2 (&S)[2][2][256]) {
#pragma unroll
    for (int o = 0; o < 2; ++o) {
      const bool bytes = !((SCV >> o) & 1);
      uint32_t pr[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const uint32_t two = bytes ? rsb[o][2 * k] | (rsb[o][2 * k + 1] << 8)
                                   : (k < 2 ? rs[o].x : rs[o].y) >> (16 * (k & 1));
        pr[k] = scale_pair_f16<FMT>(two);
      }
      S[o][0][t] = make_uint2(pr[0], pr[1]);
      S[o][1][t] = make_uint2(pr[2], pr[3]);
    }
  };

  floatx16 acc[4][4];
#pragma unroll
  for (int mi = 0; mi < 4; ++mi)
#pragma unroll
    for (int ni = 0; ni < 4; ++ni) acc[mi][ni] = floatx16{};

  const int i = lane & 31, h = lane >> 5;
  uint32_t a_raw[4][8], b_raw[4][8];
  uint2 a_sc[4], b_sc[4];
  auto read_stage = [&](const uint4 (&C)[2][1024], const uint2 (&S)[2][2][256]) {
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) {
      const int row = wm * 128 + mi * 32 + i;
      const int sw = dma_swizzle(row);
      const uint4 c0 = C[0][row * 4 + ((2 * h) ^ sw)];
      const uint4 c1 = C[0][row * 4 + ((2 * h + 1) ^ sw)];
      a_raw[mi][0] = c0.x; a_raw[mi][1] = c0.y; a_raw[mi][2] = c0.z; a_raw[mi][3] = c0.w;
      a_raw[mi][4] = c1.x; a_raw[mi][5] = c1.y; a_raw[mi][6] = c1.z; a_raw[mi][7] = c1.w;
      a_sc[mi] = S[0][h][row];
    }
#pragma unroll
    for (int ni = 0; ni < 4; ++ni) {
      const int row = wn * 128 + ni * 32 + i;
      const int sw = dma_swizzle(row);
      const uint4 c0 = C[1][row * 4 + ((2 * h) ^ sw)];
      const uint4 c1 = C[1][row * 4 + ((2 * h + 1) ^ sw)];
      b_raw[ni][0] = c0.x; b_raw[ni][1] = c0.y; b_raw[ni][2] = c0.z; b_raw[ni][3] = c0.w;
      b_raw[ni][4] = c1.x; b_raw[ni][5] = c1.y; b_raw[ni][6] = c1.z; b_raw[ni][7] = c1.w;
      b_sc[ni] = S[1][h][row];
    }
  };

  // Step s on stage C (raw codes and scales already in registers) while the
  // next step (s + 1, or s again on the last step: the other stage is not
  // read afterwards) fills stage N: its scale loads and code DMA are issued
  // at the top; after slice 6 the DMA has landed and the decoded scales are
  // stored (one wait for both), then the barrier, and the next stage's LDS
  // reads overlap slice 7.  N was last read before the previous barrier.
  auto step = [&](uint4 (&Nc)[2][1024], uint2 (&Ns)[2][2][256], int s) {
    const int nxt = s + 1 < nsteps ? s + 1 : s;
    load_scales(nxt);
    dma_codes_nv(Nc, src, nxt, wave);
    __builtin_amdgcn_sched_barrier(0);     // keep the loads at the top of the step
    Frag f0, f1;
    dequant_slice<0>(f0, a_raw, b_raw, a_sc, b_sc);
    pipelined_slice<0>(acc, f0, f1, a_raw, b_raw, a_sc, b_sc);
    pipelined_slice<1>(acc, f1, f0, a_raw, b_raw, a_sc, b_sc);
    pipelined_slice<2>(acc, f0, f1, a_raw, b_raw, a_sc, b_sc);
    pipelined_slice<3>(acc, f1, f0, a_raw, b_raw, a_sc, b_sc);
    pipelined_slice<4>(acc, f0, f1, a_raw, b_raw, a_sc, b_sc);
    pipelined_slice<5>(acc, f1, f0, a_raw, b_raw, a_sc, b_sc);
    pipelined_slice<6>(acc, f0, f1, a_raw, b_raw, a_sc, b_sc);
    wait_vmcnt<0>();
    store_scales(Ns);
    __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4));   // this wave's LDS stores done
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    read_stage(Nc, Ns);
    pipelined_slice<7>(acc, f1, f0, a_raw, b_raw, a_sc, b_sc);
  };

  load_scales(0);
  dma_codes_nv(cst0, src, 0, wave);
  store_scales(sst0);
  wait_vmcnt<0>();
  ring_barrier();
  read_stage(cst0, sst0);
  for (int s = 0; s < nsteps; s += 2) {
    step(cst1, sst1, s);
    step(cst0, sst0, s + 1);
  }

  float scale = FMT == kUE ? 1024.0f : 1.0f;   // undo the two 2^-5 scale shifts
  if (p.s_dec[0]) scale *= *p.s_dec[0];
  const float sb = p.s_dec[1] ? *p.s_dec[1] : 1.0f;
#pragma unroll
  for (int mi = 0; mi < 4; ++mi)
#pragma unroll
    for (int ni = 0; ni < 4; ++ni) acc[mi][ni] *= scale;
  epilogue(p, acc, sb, m0, n0, wm, wn, lane);
}

}  // namespace

namespace fp4lib {

// One past the largest scale byte offset a GEMM operand of `rows` rows reads.
static int64_t scale_extent(const Params& p, int o, int64_t rows) {
  const int64_t kb = p.K / 16;    // an upper bound on K-blocks for every format
  if (p.tiled[o]) return ((rows + 255) / 256) * p.kg * 2048;
  return ((rows - 1) >> p.rg_shift[o]) * p.s_row[o] + kb * p.s_kblk[o] + 1;
}

// LDS beyond the default 64 KiB must be opted into once per kernel and
// device; remember which (device, kernel) pairs are done (setting it twice
// is harmless, so a racing first call is too).
static hipError_t launch_kernel(void (*kernel)(Params), size_t lds, int grid, hipStream_t s,
                                const Params& p) {
  constexpr int kSlots = 64;
  static const void* done_fn[kSlots];
  static int done_dev[kSlots];
  static int n_done = 0;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  bool found = false;
  for (int i = 0; i < n_done && !found; ++i)
    found = done_fn[i] == reinterpret_cast<const void*>(kernel) && done_dev[i] == dev;
  if (!found) {
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(kernel),
                            hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
    if (e != hipSuccess) return e;
    if (n_done < kSlots) {
      done_fn[n_done] = reinterpret_cast<const void*>(kernel);
      done_dev[n_done] = dev;
      ++n_done;
    }
  }
  hipLaunchKernelGGL(kernel, dim3(grid), dim3(kThreads), lds, s, p);
  return hipSuccess;
}

hipError_t launch_gemm(int format, const GemmOperand& A, const GemmOperand& B, int64_t M,
                       int64_t N, int64_t K, float* D, int64_t ldd, int accumulate,
                       hipStream_t s) {
  Params p{};
  const GemmOperand* ops[2] = {&A, &B};
  for (int o = 0; o < 2; ++o) {
    p.codes[o] = ops[o]->codes;
    p.ld[o] = ops[o]->ld_codes;
    p.scales[o] = ops[o]->scales;
    p.s_row[o] = ops[o]->s_row;
    p.s_kblk[o] = ops[o]->s_kblk;
    p.rg_shift[o] = ops[o]->row_group == 16 ? 4 : 0;
    p.vec16[o] = (ops[o]->ld_codes % 16 == 0) &&
                 (reinterpret_cast<uintptr_t>(ops[o]->codes) % 16 == 0);
    // 8 (two-level) or 4 (MXFP4) scale bytes per row and K step
    const int sv = format == FP4_MXFP4 ? 4 : 8;
    p.tiled[o] = ops[o]->tiled ? 1 : 0;
    if (p.tiled[o]) p.s_kblk[o] = 1;
    p.sc_vec[o] = p.tiled[o] || (ops[o]->s_kblk == 1 && ops[o]->s_row % sv == 0 &&
                                 reinterpret_cast<uintptr_t>(ops[o]->scales) % sv == 0);
    p.s_dec[o] = format == FP4_MXFP4 ? nullptr : ops[o]->s_dec;
  }
  p.D = D;
  p.ldd = ldd;
  p.M = M;
  p.N = N;
  p.K = K;
  p.accumulate = accumulate;
  p.kg = (K / (format == FP4_MXFP4 ? 32 : 16) + 7) / 8;
  p.tiles_m = static_cast<int>((M + kBM - 1) / kBM);
  p.tiles_n = static_cast<int>((N + kBN - 1) / kBN);
  const int grid = p.tiles_m * p.tiles_n;
  if (grid == 0) return hipSuccess;
  const bool fast = M % kBM == 0 && N % kBN == 0 && p.vec16[0] && p.vec16[1] &&
                    K % (format == FP4_MXFP4 ? kBKX : kBK2) == 0;
  const int scv = (p.sc_vec[0] ? 1 : 0) | (p.sc_vec[1] ? 2 : 0);
  void (*kern)(Params) = nullptr;
  size_t lds;
  // LDS-DMA ring: whole turns of the ring, contiguous 4-byte-aligned scale rows
  const bool ring = format == FP4_MXFP4 && K > 0 && K % (kStagesX * kBKX) == 0 && p.vec16[0] && p.vec16[1] &&
                    p.sc_vec[0] && p.sc_vec[1];
  if (ring && p.tiled[0] && p.tiled[1]) {
    hipLaunchKernelGGL(k_gemm_mx_tiled, dim3(grid), dim3(kThreads), 0, s, p);
    return hipGetLastError();
  }
  if (ring) {
    hipLaunchKernelGGL(k_gemm_mx_ring, dim3(grid), dim3(kThreads), 0, s, p);
    return hipGetLastError();
  }
  if (format == FP4_MXFP4) {
    lds = 2 * sizeof(StageX);
    constexpr void (*mx[4])(Params) = {k_gemm_mx<true, 0>, k_gemm_mx<true, 1>,
                                       k_gemm_mx<true, 2>, k_gemm_mx<true, 3>};
    kern = fast ? mx[scv] : k_gemm_mx<false, 0>;
  } else if (format == FP4_NVFP4 && K > 0 && K % (2 * kBK2) == 0 && p.vec16[0] && p.vec16[1] &&
             M * p.ld[0] < (int64_t(1) << 31) && N * p.ld[1] < (int64_t(1) << 31) &&
             scale_extent(p, 0, M) < (int64_t(1) << 31) &&
             scale_extent(p, 1, N) < (int64_t(1) << 31)) {
    // NVFP4 codes by DMA: whole pairs of K steps, 16-byte code rows.  (UE5M3
    // stays on the register-staged kernel: its arithmetic scale decode sits
    // in front of this kernel's barrier and costs more than the DMA saves.)
    constexpr void (*dnv[4])(Params) = {k_gemm_two_level_dma<kNV, 0>, k_gemm_two_level_dma<kNV, 1>,
                                        k_gemm_two_level_dma<kNV, 2>, k_gemm_two_level_dma<kNV, 3>};
    hipLaunchKernelGGL(dnv[scv], dim3(grid), dim3(kThreads), 0, s, p);
    return hipGetLastError();
  } else if (format == FP4_NVFP4) {
    lds = 2 * sizeof(Stage2);
    constexpr void (*nv[4])(Params) = {k_gemm_two_level<kNV, true, 0>, k_gemm_two_level<kNV, true, 1>,
                                       k_gemm_two_level<kNV, true, 2>, k_gemm_two_level<kNV, true, 3>};
    kern = fast ? nv[scv] : k_gemm_two_level<kNV, false, 0>;
  } else {
    lds = 2 * sizeof(Stage2);
    constexpr void (*ue[4])(Params) = {k_gemm_two_level<kUE, true, 0>, k_gemm_two_level<kUE, true, 1>,
                                       k_gemm_two_level<kUE, true, 2>, k_gemm_two_level<kUE, true, 3>};
    kern = fast ? ue[scv] : k_gemm_two_level<kUE, false, 0>;
  }
  const hipError_t e = launch_kernel(kern, lds, grid, s, p);
  if (e != hipSuccess) return e;
  return hipGetLastError();
}

}  // namespace fp4lib
