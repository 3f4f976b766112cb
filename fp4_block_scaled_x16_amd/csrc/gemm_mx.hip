// MXFP4 block-scaled GEMM on the scaled FP4 MFMA with register-staged codes:
// every shape (ragged M, N and K tails masked).

#include "gemm_common.hpp"

namespace fp4gemm {
namespace {

// -------------------------------------------------------------- MXFP4 ---

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

}  // namespace

hipError_t launch_mx(bool fast, int scv, const Params& p, int grid, hipStream_t s) {
  constexpr void (*mx[4])(Params) = {k_gemm_mx<true, 0>, k_gemm_mx<true, 1>,
                                     k_gemm_mx<true, 2>, k_gemm_mx<true, 3>};
  return launch_with_lds(fast ? mx[scv] : k_gemm_mx<false, 0>, 2 * sizeof(StageX), grid, s, p);
}

}  // namespace fp4gemm
