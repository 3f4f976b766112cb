// NVFP4 / UE5M3 block-scaled GEMM with the codes moved into LDS by DMA (K a
// multiple of 256, 16-byte-aligned code rows).  This source is compiled once
// per (format, tile height) with FP4_DMA_FMT (0 NVFP4, 1 UE5M3) and
// FP4_DMA_MI (4: 256-row tiles, 3: 192-row tiles) defined, so the four
// kernel families build in parallel; each object defines one launcher.

#include "gemm_common.hpp"

namespace fp4gemm {
namespace {

// ------------------------------------------- NVFP4 / UE5M3, codes by DMA ---
// The two-level product for K a multiple of 256 and 16-byte-aligned code
// rows: the same per-lane dequantization and slice pipeline as
// k_gemm_two_level, but the codes go from global memory straight into LDS
// (global_load_lds, 16 bytes per lane) instead of through registers and LDS
// stores, and ragged M / N read the last valid row (never stored).  Block
// scales are still loaded to registers and decoded once per K step by the
// loading thread, off the path to the barrier (see the step below).  Codes and scales of each of the two stages are separate
// __shared__ variables named with compile-time indices, so the compiler can
// tell the DMA targets from the LDS the waves read and write.
//
// MI is the number of 32-row MFMA tiles per wave in M: 4 gives the usual
// 256 x 256 tile, 3 a 192 x 256 tile (each wave 96 x 128), for shapes where
// 256-row tiles would leave part of the chip idle in the last round (e.g.
// 6144 output rows: 192 tiles of 256 rows on 256 CUs, but 256 of 192 rows).
struct DmaSrcNv {
  const uint8_t* base[2];       // operand code matrices (uniform)
  uint32_t off[2][4];           // this lane's 16 bytes of rows wave*(16 J) + 16j + lane/4
};                              // (the host keeps every offset below 2^31)

// Operand o's tile has 64 J rows (J = MI for A, 4 for B); wave w loads rows
// 16 J w .. 16 J w + 16 J - 1, 16 rows per instruction.
template <int MI>
__device__ __forceinline__ void dma_codes_nv(uint4 (&dst)[2][1024], const DmaSrcNv& src,
                                             int64_t step, int wave) {
  const int64_t cb = step * (kBK2 / 2);
#pragma unroll
  for (int o = 0; o < 2; ++o) {
    constexpr int J[2] = {MI, 4};
#pragma unroll
    for (int j = 0; j < J[o]; ++j)
      __builtin_amdgcn_global_load_lds(src.base[o] + cb + src.off[o][j],
                                       &dst[o][wave * (64 * J[o]) + j * 64], 16, 0, 0);
  }
}

// Scheduling hint for the last slice of a step: the stage's LDS reads go
// first, then a quarter of the slice's MFMAs alone (the reads land
// meanwhile), then the rest each followed by its share of the next step's
// slice-0 dequantization.
template <int MI>
__device__ __forceinline__ void interleave_tail() {
  constexpr int kReads = 2 * (MI + 4) + (MI + 4);   // 16-byte code reads + scale reads
  constexpr int kFirst = MI;
  constexpr int kRest = 4 * MI - kFirst;
  constexpr int kValu = (8 * (MI + 4) + kRest - 1) / kRest;
  __builtin_amdgcn_sched_group_barrier(0x100, kReads, 0);   // DS read
  __builtin_amdgcn_sched_group_barrier(0x008, kFirst, 0);   // MFMA
#pragma unroll
  for (int i = 0; i < kRest; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);      // MFMA
    __builtin_amdgcn_sched_group_barrier(0x002, kValu, 0);  // VALU
  }
}

template <int FMT, int SCV, int MI>
__global__ __launch_bounds__(kThreads, 1) void k_gemm_two_level_dma(Params p) {
  constexpr int BM = 64 * MI;
  __shared__ uint4 cst0[2][1024], cst1[2][1024];   // [operand][row * 4 + (chunk ^ swizzle)]
  __shared__ uint2 sst0[2][2][256], sst1[2][2][256];  // [operand][half][row] fp16 scale pairs
  // per-row decode scales of the tile's A rows and B rows (per-row global
  // scales only): loaded with the first K step's scales, read by the epilogue
  __shared__ __attribute__((aligned(16))) float srow[2][256];
  __shared__ __attribute__((aligned(16))) float ept[4][2 * kEpiBufFloats];
  int tm, tn;
  tile_coords(p, tm, tn);
  const int64_t m0 = static_cast<int64_t>(tm) * BM, n0 = static_cast<int64_t>(tn) * kBN;
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
    const int J = o == 0 ? MI : 4;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int row = wave * (16 * J) + j * 16 + (lane >> 2);
      const int q = (lane & 3) ^ dma_swizzle(row);
      const int64_t r = min(base[o] + row, lim[o] - 1);
      src.off[o][j] = static_cast<uint32_t>(r * p.ld[o] + q * 16);
    }
  }
  // scales of row t (clamped), K step s: a per-lane offset plus a uniform
  // per-step stride (one 2 KiB atom TILED, 8 K-blocks otherwise).  With
  // BM < 256, threads t >= BM load and store A scales that are never read.
  uint32_t soff[2];
  int64_t sstep[2];
#pragma unroll
  for (int o = 0; o < 2; ++o) {
    soff[o] = static_cast<uint32_t>(scale_ptr(p, o, min(base[o] + t, lim[o] - 1), 0) - p.scales[o]);
    sstep[o] = p.tiled[o] ? 2048 : 8 * p.s_kblk[o];
  }

  // Raw scale bytes are loaded two K steps ahead, at the top of a step, and
  // decoded (into pr) after that step's barrier, under its last slice's
  // MFMAs, when the loads have long landed; the decoded pairs are stored
  // into the stage at the end of the next step.  So no step waits for loads
  // it has just issued, and only an LDS store sits between the code DMA's
  // arrival and the barrier.  The decode (scale_pair_f16: one instruction
  // per pair for E4M3, five for UE5M3) fills VALU slots of the last slice.
  uint2 rs[2];
  uint32_t rsb[2][8];
  uint32_t pr[2][4];
  constexpr int kScaleLoads = (SCV & 1 ? 1 : 8) + (SCV & 2 ? 1 : 8);
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
  auto decode_scales = [&]() {
#pragma unroll
    for (int o = 0; o < 2; ++o) {
      const bool bytes = !((SCV >> o) & 1);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        if (bytes)
          pr[o][k] = scale_pair_f16<FMT>(rsb[o][2 * k] | (rsb[o][2 * k + 1] << 8));
        else if (k & 1)
          pr[o][k] = scale_pair_f16<FMT, 2>(k < 2 ? rs[o].x : rs[o].y);
        else
          pr[o][k] = scale_pair_f16<FMT, 0>(k < 2 ? rs[o].x : rs[o].y);
      }
    }
  };
  auto store_scales = [&](uint2 (&S)[2][2][256]) {
#pragma unroll
    for (int o = 0; o < 2; ++o) {
      S[o][0][t] = make_uint2(pr[o][0], pr[o][1]);
      S[o][1][t] = make_uint2(pr[o][2], pr[o][3]);
    }
  };

  floatx16 acc[MI][4];
#pragma unroll
  for (int mi = 0; mi < MI; ++mi)
#pragma unroll
    for (int ni = 0; ni < 4; ++ni) acc[mi][ni] = floatx16{};

  const int i = lane & 31, h = lane >> 5;
  uint32_t a_raw[MI][8], b_raw[4][8];
  uint2 a_sc[MI], b_sc[4];
  // LDS reads of a stage into the raw-code and scale registers, in the
  // order the slices need them: the first 16 bytes of every row (slices
  // 0-3) and the scales first, the second 16 bytes (slices 4-7) last.
  auto read_stage = [&](const uint4 (&C)[2][1024], const uint2 (&S)[2][2][256]) {
    auto read_half = [&](int q) {
#pragma unroll
      for (int mi = 0; mi < MI; ++mi) {
        const int row = wm * (MI * 32) + mi * 32 + i;
        const uint4 c = C[0][row * 4 + ((2 * h + q) ^ dma_swizzle(row))];
        a_raw[mi][4 * q] = c.x; a_raw[mi][4 * q + 1] = c.y;
        a_raw[mi][4 * q + 2] = c.z; a_raw[mi][4 * q + 3] = c.w;
      }
#pragma unroll
      for (int ni = 0; ni < 4; ++ni) {
        const int row = wn * 128 + ni * 32 + i;
        const uint4 c = C[1][row * 4 + ((2 * h + q) ^ dma_swizzle(row))];
        b_raw[ni][4 * q] = c.x; b_raw[ni][4 * q + 1] = c.y;
        b_raw[ni][4 * q + 2] = c.z; b_raw[ni][4 * q + 3] = c.w;
      }
    };
    read_half(0);
#pragma unroll
    for (int mi = 0; mi < MI; ++mi) a_sc[mi] = S[0][h][wm * (MI * 32) + mi * 32 + i];
#pragma unroll
    for (int ni = 0; ni < 4; ++ni) b_sc[ni] = S[1][h][wn * 128 + ni * 32 + i];
    read_half(1);
  };

  // Step s on stage C (raw codes and scales already in registers) while the
  // next step (s + 1, or s again on the last step: the other stage is not
  // read afterwards) fills stage N.  At the top: the code DMA of step s + 1,
  // then the scale loads of step s + 2.  After slice 6 the DMA has landed
  // (the younger scale loads may still be in flight), the scales of step
  // s + 1 (decoded during step s - 1) are stored, then the barrier; the next
  // stage's LDS reads and the decode of step s + 2's scales overlap slice
  // 7.  N was last read before the previous barrier.  Slice 0 of a step is
  // dequantized either at the top of the step (256-row tiles) or, for
  // 192-row tiles, under the second part of the previous step's slice 7
  // (kTail; measured faster there, slower with 256 rows, whose slice-7
  // MFMAs cannot hide the 8 extra VALU ops per MFMA).
  constexpr bool kTail = MI != 4;
  FragT<MI> f0, f1;
  auto step = [&](uint4 (&Nc)[2][1024], uint2 (&Ns)[2][2][256], int s) {
    const int nxt = s + 1 < nsteps ? s + 1 : s;
    const int nxt2 = s + 2 < nsteps ? s + 2 : nsteps - 1;
    dma_codes_nv<MI>(Nc, src, nxt, wave);
    __builtin_amdgcn_sched_barrier(0);     // the DMA is issued before (is older than) ...
    load_scales(nxt2);                     // ... the scale loads: the vmcnt wait relies on it
    __builtin_amdgcn_sched_barrier(0);     // keep the loads at the top of the step
    if constexpr (!kTail) dequant_slice<0>(f0, a_raw, b_raw, a_sc, b_sc);
    pipelined_slice<0>(acc, f0, f1, a_raw, b_raw, a_sc, b_sc);
    pipelined_slice<1>(acc, f1, f0, a_raw, b_raw, a_sc, b_sc);
    pipelined_slice<2>(acc, f0, f1, a_raw, b_raw, a_sc, b_sc);
    pipelined_slice<3>(acc, f1, f0, a_raw, b_raw, a_sc, b_sc);
    pipelined_slice<4>(acc, f0, f1, a_raw, b_raw, a_sc, b_sc);
    pipelined_slice<5>(acc, f1, f0, a_raw, b_raw, a_sc, b_sc);
    pipelined_slice<6>(acc, f0, f1, a_raw, b_raw, a_sc, b_sc);
    // Nothing crosses these fences: without them the scheduler lifts the
    // wait, the store and the barrier (which the MFMAs do not depend on)
    // above the slices, and every step would stall on the DMA it has just
    // issued.
    __builtin_amdgcn_sched_barrier(0);
    wait_vmcnt<kScaleLoads>();              // the code DMA of step s + 1
    store_scales(Ns);
    __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4));   // this wave's LDS stores done
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    read_stage(Nc, Ns);
    wait_vmcnt<0>();                        // step s + 2's scale bytes (issued at the top)
    decode_scales();
    if constexpr (kTail) {
      dequant_slice<0>(f0, a_raw, b_raw, a_sc, b_sc);
      mfma_slice(acc, f1);
      interleave_tail<MI>();
    } else {
      pipelined_slice<7>(acc, f1, f0, a_raw, b_raw, a_sc, b_sc);
    }
  };

  float srow_v[2] = {1.0f, 1.0f};
#pragma unroll
  for (int o = 0; o < 2; ++o)
    if (p.s_dec_rows[o]) srow_v[o] = p.s_dec[o][min(base[o] + t, lim[o] - 1)];
  load_scales(0);
  dma_codes_nv<MI>(cst0, src, 0, wave);
  wait_vmcnt<0>();
  decode_scales();
  store_scales(sst0);
#pragma unroll
  for (int o = 0; o < 2; ++o)
    if (p.s_dec_rows[o]) srow[o][t] = srow_v[o];
  load_scales(nsteps > 1 ? 1 : 0);       // step 1's scales, stored at the end of step 0
  wait_vmcnt<0>();
  decode_scales();
  ring_barrier();
  read_stage(cst0, sst0);
  if constexpr (kTail) dequant_slice<0>(f0, a_raw, b_raw, a_sc, b_sc);
  for (int s = 0; s < nsteps; s += 2) {
    step(cst1, sst1, s);
    step(cst0, sst0, s + 1);
  }
  wait_vmcnt<0>();                         // the last (unused) scale loads

  float scale = FMT == kUE ? 1024.0f : 1.0f;   // undo the two 2^-5 scale shifts
  if (p.s_dec[0] && !p.s_dec_rows[0]) scale *= *p.s_dec[0];
  const float sb = p.s_dec[1] && !p.s_dec_rows[1] ? *p.s_dec[1] : 1.0f;
  if (epilogue_lds_ok<MI, MI == 3>(p, m0, n0, wm, wn)) {
    epilogue_lds<MI, 2, MI == 3>(p, acc, scale, sb, m0, n0, wm, wn, lane, ept[wave]);
  } else {
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
      for (int ni = 0; ni < 4; ++ni) acc[mi][ni] *= scale;
    epilogue(p, acc, sb, m0, n0, wm, wn, lane, srow[0], srow[1]);
  }
}

}  // namespace

#if !defined(FP4_DMA_FMT) || !defined(FP4_DMA_MI)
#error "compile with -DFP4_DMA_FMT=0|1 -DFP4_DMA_MI=4|3"
#endif

// This object's launcher, launch_two_level_dma_<FMT>_<MI>: scale-loader
// variant `scv` (bit o: operand o's scales of one row and K step are one
// aligned 8-byte word).
#define FP4_DMA_NAME2(f, m) launch_two_level_dma_##f##_##m
#define FP4_DMA_NAME(f, m) FP4_DMA_NAME2(f, m)
hipError_t FP4_DMA_NAME(FP4_DMA_FMT, FP4_DMA_MI)(int scv, const Params& p, hipStream_t s) {
  constexpr int F = FP4_DMA_FMT == 0 ? kNV : kUE;
  constexpr void (*k[4])(Params) = {
      k_gemm_two_level_dma<F, 0, FP4_DMA_MI>, k_gemm_two_level_dma<F, 1, FP4_DMA_MI>,
      k_gemm_two_level_dma<F, 2, FP4_DMA_MI>, k_gemm_two_level_dma<F, 3, FP4_DMA_MI>};
  hipLaunchKernelGGL(k[scv], dim3(p.tiles_m * p.tiles_n), dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace fp4gemm
