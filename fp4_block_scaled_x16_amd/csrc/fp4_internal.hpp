// Internal launch interface between the C ABI (fp4_api.cpp) and the kernel
// translation units.  Arguments have been validated by the caller.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/fp4.h"
#include "../../include/fp4_selftest.h"

namespace fp4lib {

struct QuantArgs {
  const uint16_t* x;
  int64_t rows, cols, ld;
  uint8_t* codes;
  uint8_t* scales;
  uint8_t* codes_t;
  const float* amax;     // device; read by the quantize kernel (MXFP4: unused);
                         // per-row scope: float[rows], written unless amax_given
  float* s_dec;          // device or null
  fp4_counters* counters;
  float target;
  uint64_t seed, offset;
  uint32_t rht_signs[4];   // D_r of the RHT: bit i negates output row i (128 bits)
  int rht_n;               // RHT size: 4, 16, 32, 64 or 128 (0 means 16)
  int format, round, rht, emit_transpose;
  int tiled;             // 1D scales in the TILED layout (2 KiB atoms of 256 rows x 8 blocks)
  int scale_up;          // block scales rounded up (truncation-free), two-level formats
  int amax_given;        // per-row scope: read amax[r] instead of computing it
  int count_elems;       // with counters: element events too (else block-scale events only)
};

struct GemmOperand {
  const uint8_t* codes;
  int64_t ld_codes;
  const uint8_t* scales;
  int64_t s_row, s_kblk;
  int row_group;
  const float* s_dec;
  bool tiled;            // scales in the TILED layout (strides unused)
  bool s_dec_rows;       // s_dec holds one decode scale per operand row
};

// Number of compute units of the current device (cached per device).
int device_cu_count();
// Workgroups of a persistent grid of per_cu workgroups per CU, capped by the
// launch-geometry control (fp4_selftest_set_geometry) when one is set.
int64_t grid_cap(int per_cu);
// Forced tile height of the two-level DMA GEMM (192 or 256), 0 if none.
int gemm_tile_rows_forced();
void set_launch_geometry(int max_workgroups, int gemm_tile_rows);

// amax_plain (optional, rht with N = 16 along the columns only): also max |x|
// from the same read.  along_rows: the rotation runs along the rows of x
// (rowwise quantization) instead of along its columns.
hipError_t launch_amax(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld, int rht,
                       int rht_n, const uint32_t (&signs)[4], float* amax, hipStream_t s,
                       float* amax_plain = nullptr, bool along_rows = false);
hipError_t launch_quant_row(const QuantArgs& a, hipStream_t s);
// Rowwise 1D with one global scale per row (two-level formats): the row
// amaxes (a.amax, float[rows]) come from the same read that quantizes.
hipError_t launch_quant_row_scoped(const QuantArgs& a, hipStream_t s);
hipError_t launch_quant_col(const QuantArgs& a, hipStream_t s);
// MXFP8 (E4M3 elements, 1x32 blocks, UE8M0 scales), rowwise or colwise.
hipError_t launch_quant_mx8(const QuantArgs& a, bool colwise, hipStream_t s);
hipError_t launch_dequant_mx8(int tiled, const uint8_t* codes, const uint8_t* scales, int64_t rows,
                              int64_t cols, void* out, int out_fp32, hipStream_t s);
hipError_t launch_quant_2d(const QuantArgs& a, hipStream_t s);
// Rowwise (`row`) and colwise (`col`) 1D quantization of the same input in
// one kernel: same format and rounding mode; RHT only on the colwise side.
hipError_t launch_quant_dual(const QuantArgs& row, const QuantArgs& col, hipStream_t s);
// s_dec_rows: s_dec holds one decode scale per row.
hipError_t launch_dequant(int format, int block2d, int tiled, const uint8_t* codes,
                          const uint8_t* scales, const float* s_dec, bool s_dec_rows,
                          int64_t rows, int64_t cols, void* out, int out_fp32, hipStream_t s);
// The RHT of size rht_n (0 means 16) alone, along the rows or the columns.
hipError_t launch_rht(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld, int rht_n,
                      const uint32_t (&signs)[4], bool along_rows, float* y, hipStream_t s);
hipError_t launch_gemm(int format, const GemmOperand& A, const GemmOperand& B, int64_t M, int64_t N,
                       int64_t K, void* D, int d_bf16, int64_t ldd, int accumulate,
                       hipStream_t s);
// Exhaustive conversion checks (selftest.hip).
hipError_t launch_selftest_sweep(int kind, const uint32_t* thresholds, int n, uint64_t* result,
                                 hipStream_t s);
hipError_t launch_selftest_gemm_decode(int format, uint16_t* out, hipStream_t s);

}  // namespace fp4lib
