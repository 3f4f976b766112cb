// Block-scaled FP4 GEMMs for gfx950 (NVFP4 pretraining paper, App. B.3:
// per-block partial products scaled by both local decode scales, fp32
// accumulation, the two global decode scales applied to the output; §4.1 /
// Fig. 5: Fprop, Dgrad and Wgrad all run this product on FP4 operands).
//
//   D[M, N] (+)= s_A s_B sum_k a[m, k] b[n, k],   a = e2m1 * scale ("TN")
//
// Every kernel uses one skeleton: a 256 x 256 output tile per workgroup
// (192 x 256 for some NVFP4 / UE5M3 shapes),
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
//     k_gemm_two_level_dma  K % 256 == 0, 16-byte code rows: codes go to
//                           LDS by DMA (global_load_lds); 256- or 192-row
//                           tiles (gemm_nv_dma.hip).
//     k_gemm_two_level      every other shape: codes staged through
//                           registers, ragged edges masked (gemm_nv.hip).
// * MXFP4: gfx950's scaled MFMA takes FP4 operands and one E8M0 scale per 32
//   K-values per lane, which is exactly an MXFP4 block, so the codes go from
//   LDS to v_mfma_scale_f32_32x32x64_f8f6f4 untouched.
//     k_gemm_mx_tiled  TILED scales, K % 512 == 0: K step 256, codes and
//                      scales by DMA in whole 128-byte lines.
//     k_gemm_mx_ring   K % 512 == 0, other scale layouts: 4-stage K-128 DMA ring.
//     k_gemm_mx        every other shape: register-staged, edges masked
//                      (gemm_mx.hip; the two DMA kernels: gemm_mx_dma.hip).
//
// The order of K inside one K step is free as long as A and B agree: lane
// half h of a wave owns a contiguous half of the step's K range for both
// operands, so each lane's codes are one contiguous run in LDS.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fp4_internal.hpp"
#include "gemm_common.hpp"

namespace fp4gemm {

// LDS beyond the default 64 KiB must be opted into once per kernel and
// device; remember which (device, kernel) pairs are done (setting it twice
// is harmless, so a racing first call is too).
hipError_t launch_with_lds(void (*kernel)(Params), size_t lds, int grid, hipStream_t s,
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
  return hipGetLastError();
}

}  // namespace fp4gemm

namespace fp4lib {

using fp4gemm::Params;

// One past the largest scale byte offset a GEMM operand of `rows` rows reads.
static int64_t scale_extent(const Params& p, int o, int64_t rows) {
  const int64_t kb = p.K / 16;    // an upper bound on K-blocks for every format
  if (p.tiled[o]) return ((rows + 255) / 256) * p.kg * 2048;
  return ((rows - 1) >> p.rg_shift[o]) * p.s_row[o] + kb * p.s_kblk[o] + 1;
}

hipError_t launch_gemm(int format, const GemmOperand& A, const GemmOperand& B, int64_t M,
                       int64_t N, int64_t K, void* D, int d_bf16, int64_t ldd, int accumulate,
                       hipStream_t s) {
  using namespace fp4gemm;
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
    p.s_dec_rows[o] = p.s_dec[o] && ops[o]->s_dec_rows ? 1 : 0;
  }
  p.D = static_cast<float*>(D);
  p.d_bf16 = d_bf16;
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
  if (format == FP4_MXFP4) {
    // LDS-DMA kernels: whole turns of the ring, contiguous 4-byte-aligned scale rows
    const bool ring = K > 0 && K % (kStagesX * kBKX) == 0 && p.vec16[0] && p.vec16[1] &&
                      p.sc_vec[0] && p.sc_vec[1];
    if (ring && p.tiled[0] && p.tiled[1]) return launch_mx_tiled(p, grid, s);
    if (ring) return launch_mx_ring(p, grid, s);
    return launch_mx(fast, scv, p, grid, s);
  }
  if (K > 0 && K % (2 * kBK2) == 0 && p.vec16[0] && p.vec16[1] &&
      M * p.ld[0] < (int64_t(1) << 31) && N * p.ld[1] < (int64_t(1) << 31) &&
      scale_extent(p, 0, M) < (int64_t(1) << 31) && scale_extent(p, 1, N) < (int64_t(1) << 31)) {
    // Codes by DMA: whole pairs of K steps, 16-byte code rows.  Tile height
    // 192 instead of 256 when that shortens the launch: its time goes as (rounds of tiles over the CUs) x (tile height), with a
    // 5 % allowance for the smaller tile's lower MFMA share per VALU op.
    const int64_t cus = device_cu_count();
    auto cost = [&](int64_t bm) {
      const int64_t tiles = (M + bm - 1) / bm * p.tiles_n;
      return (tiles + cus - 1) / cus * bm;
    };
    const int forced = gemm_tile_rows_forced();
    const int short_tile = forced ? (forced == 192 ? 1 : 0) : (cost(192) * 20 < cost(256) * 19 ? 1 : 0);
    if (short_tile) p.tiles_m = static_cast<int>((M + 191) / 192);
    if (format == FP4_NVFP4)
      return short_tile ? launch_two_level_dma_0_3(scv, p, s) : launch_two_level_dma_0_4(scv, p, s);
    return short_tile ? launch_two_level_dma_1_3(scv, p, s) : launch_two_level_dma_1_4(scv, p, s);
  }
  return format == FP4_NVFP4 ? launch_two_level_0(fast, scv, p, grid, s)
                             : launch_two_level_1(fast, scv, p, grid, s);
}

}  // namespace fp4lib
