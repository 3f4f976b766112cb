// MXFP4 block-scaled GEMMs with codes and scales moved into LDS by DMA:
// the K-128 four-stage ring (any 1D scale layout) and the K-256 kernel for
// TILED scales.  Both need K a multiple of 512.

#include "gemm_common.hpp"

namespace fp4gemm {
namespace {

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
constexpr int kDmaPerStep = 10;   // per wave: 2 x 4 code chunks + 2 scale rows

struct StageD {
  uint4 codes[2][1024];     // [operand][row * 4 + (chunk ^ dma_swizzle(row))]
  uint32_t scales[2][256];  // [operand][row]: E8M0 bytes of the step's 4 blocks
};

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
  // every wave is past its last stage read and its DMAs have landed: stage
  // 0 holds the epilogue's per-wave transpose buffers (one each: a stage is
  // 34 KiB)
  ring_barrier();
  static_assert(sizeof(StageD) >= 4 * kEpiBufFloats * sizeof(float), "epilogue buffers");
  if (epilogue_lds_ok<4, false>(p, m0, n0, wm, wn))
    epilogue_lds<4, 1, false>(p, acc, 1.0f, 1.0f, m0, n0, wm, wn, lane,
                       reinterpret_cast<float*>(&st0) + wave * kEpiBufFloats);
  else
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
  // every wave is past its last stage read and its DMAs have landed: stage
  // 0 holds the epilogue's per-wave transpose buffers
  ring_barrier();
  static_assert(sizeof(StageV) >= 4 * 2 * kEpiBufFloats * sizeof(float), "epilogue buffers");
  if (epilogue_lds_ok<4, false>(p, m0, n0, wm, wn))
    epilogue_lds<4, 2, false>(p, acc, 1.0f, 1.0f, m0, n0, wm, wn, lane,
                       reinterpret_cast<float*>(&sv0) + wave * 2 * kEpiBufFloats);
  else
    epilogue(p, acc, 1.0f, m0, n0, wm, wn, lane);
}

}  // namespace

hipError_t launch_mx_ring(const Params& p, int grid, hipStream_t s) {
  hipLaunchKernelGGL(k_gemm_mx_ring, dim3(grid), dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_mx_tiled(const Params& p, int grid, hipStream_t s) {
  hipLaunchKernelGGL(k_gemm_mx_tiled, dim3(grid), dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace fp4gemm
