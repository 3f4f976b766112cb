// NVFP4 / UE5M3 block-scaled GEMM with register-staged codes: the shapes the
// DMA kernel does not take (ragged M, N and K tails masked).  Compiled once
// per block-scale format (FP4_NV_FMT) so the two build in parallel.

#include "gemm_common.hpp"

namespace fp4gemm {
namespace {

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
  if (p.s_dec[0] && !p.s_dec_rows[0]) scale *= *p.s_dec[0];
  // s_B is applied as a second multiply so that s_A * s_B never under/overflows alone
  const float sb = p.s_dec[1] && !p.s_dec_rows[1] ? *p.s_dec[1] : 1.0f;
#pragma unroll
  for (int mi = 0; mi < 4; ++mi)
#pragma unroll
    for (int ni = 0; ni < 4; ++ni) acc[mi][ni] *= scale;
  epilogue(p, acc, sb, m0, n0, wm, wn, lane);
}

}  // namespace

#if !defined(FP4_NV_FMT)
#error "compile with -DFP4_NV_FMT=0|1"
#endif

// This object's launcher, launch_two_level_<FMT> (0 NVFP4, 1 UE5M3): the
// tile-aligned kernel for scale-loader variant `scv` when `fast`, else the
// masked one.
#define FP4_NV_NAME2(f) launch_two_level_##f
#define FP4_NV_NAME(f) FP4_NV_NAME2(f)
hipError_t FP4_NV_NAME(FP4_NV_FMT)(bool fast, int scv, const Params& p, int grid, hipStream_t s) {
  constexpr int F = FP4_NV_FMT == 0 ? kNV : kUE;
  constexpr void (*k[4])(Params) = {k_gemm_two_level<F, true, 0>, k_gemm_two_level<F, true, 1>,
                                    k_gemm_two_level<F, true, 2>, k_gemm_two_level<F, true, 3>};
  void (*kern)(Params) = fast ? k[scv] : k_gemm_two_level<F, false, 0>;
  return launch_with_lds(kern, 2 * sizeof(Stage2), grid, s, p);
}

}  // namespace fp4gemm
