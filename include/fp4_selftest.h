/*
 * fp4_selftest.h -- exhaustive device checks of the conversions the hot
 * path of libfp4_mi355x.so relies on, exported so a test can run them on
 * the GPU against expected values it computes elsewhere (the library holds
 * no expected values of its own).
 *
 * Conversions covered (NVFP4 pretraining paper, arXiv:2509.25149):
 *  - fp32 -> E2M1 by round to nearest even, saturating at 6 (§3 value set,
 *    App. B.3 Eq. 4), exactly as the quantizer kernels call gfx950's packed
 *    FP4 convert: two values per call, written into byte 0..3 of a word;
 *  - fp32 -> E4M3 and fp32 -> UE5M3 block-scale codes by round to nearest
 *    even with saturation (App. B.2, Eq. 3; UE5M3 abstract), the encoder
 *    every two-level quantizer uses;
 *  - E2M1 code x block scale -> fp16, the GEMM's operand decode (App. B.3):
 *    gfx950's FP4 -> fp16 convert, the E4M3 scale through the FP8 -> fp16
 *    convert (UE5M3: the arithmetic decode times 2^-5), then the packed fp16
 *    multiply with either half of the scale pair broadcast.
 *
 * Conventions as in fp4.h: device pointers, work enqueued on `stream`,
 * arguments validated on the host before any HIP call, nonzero status and
 * fp4_last_error() on rejection.
 */
#ifndef FP4_MI355X_SELFTEST_H
#define FP4_MI355X_SELFTEST_H

#include <stdint.h>

#include "fp4.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef enum fp4_sweep_kind_e FP4_ENUM_INT {
  FP4_SWEEP_E2M1_RNE = 0,     /* every fp32 pattern except NaNs (2^32 - 2^24 + 2)   */
  FP4_SWEEP_E4M3_SCALE = 1,   /* every finite fp32 t >= 0 (patterns 0 .. 0x7F7FFFFF) */
  FP4_SWEEP_UE5M3_SCALE = 2,  /* likewise                                            */
  FP4_SWEEP_E2M1_SR = 3,      /* every fp32 pattern except NaNs, four draws each     */
  FP4_SWEEP_E4M3_ELEM = 4     /* every fp32 magnitude 0 .. 448 (0 .. 0x43E00000)    */
} fp4_sweep_kind;

/*
 * fp4_selftest_sweep -- run one conversion on every input of its domain and
 * compare each result with a monotone step function given by `thresholds`:
 * the expected magnitude code of an input with magnitude bits m (sign bit
 * cleared) is the number of entries t with m >= t; for E2M1 the sign bit of
 * the code copies the input's sign bit.
 *   thresholds  device uint32 array, ascending fp32 bit patterns: entry i is
 *               the smallest magnitude whose code is i + 1.  Length n:
 *               7 (E2M1), 126 (E4M3, codes 1 .. 0x7E; also for
 *               FP4_SWEEP_E4M3_ELEM), 255 (UE5M3).
 *   result      device uint64[3], overwritten: [0] inputs whose code differs,
 *               [1] the smallest differing input pattern (all ones if none),
 *               [2] inputs checked.
 * FP4_SWEEP_E2M1_SR checks stochastic rounding (NVFP4 paper §4.4, the rule
 * in fp4.h under fp4_quantize) through the quantizers' 8-value helper: the
 * 7 thresholds are the E2M1 magnitudes 0.5, 1, ..., 6 (the smallest
 * magnitude whose round-down code is i + 1); each input is converted at an
 * even and at an odd element position with the random value just below and
 * at its carry threshold (16 random bits u round up iff u + floor(65536 f)
 * >= 65536), so every input counts four times in [2].
 * FP4_SWEEP_E4M3_ELEM checks the MXFP8 element encoder (E4M3 round to
 * nearest even of the scaled element, MXFP8 row of fp4.h's format list):
 * the hardware FP8 convert the quantizer packs four elements with, over
 * the magnitudes the block scale lets through (|v * 2^-e| <= 448); each
 * input t is packed as (t, -t, -t, t) and (-t, t, t, -t), the sign going
 * to bit 7 of its byte, and counts once in [2].
 */
fp4_status fp4_selftest_sweep(int kind, const uint32_t* thresholds, int n,
                              uint64_t* result, void* stream);

/*
 * fp4_selftest_gemm_decode -- the GEMM's exact operand decode for every
 * (block-scale code, E2M1 code) pair of a two-level format.
 *   format  FP4_NVFP4 (scale codes 0 .. 0x7E) or FP4_UE5M3 (0 .. 0xFF).
 *   out     device uint16 [256][4][16]: out[s][v][c] is the fp16 bit pattern
 *           the decode gives for E2M1 code c with scale code s held in half
 *           v & 1 of the scale pair (the other half holds a different code),
 *           the pair read from bytes 0-1 (v < 2) or 2-3 (v >= 2) of a word
 *           whose other bytes hold other codes; rows s beyond the format's
 *           codes are written as 0.
 */
fp4_status fp4_selftest_gemm_decode(fp4_format format, uint16_t* out, void* stream);

/*
 * fp4_selftest_set_geometry -- launch-geometry controls for race guards: no
 * result of the library may depend on them, so a test runs the same work
 * under different settings and requires bit-identical outputs.
 *   max_workgroups  > 0: every persistent grid (amax, quantizers, dequantize,
 *                   RHT) launches at most this many workgroups, each walking
 *                   more of the work; 0: the default grids.
 *   gemm_tile_rows  192 or 256: the NVFP4 / UE5M3 DMA GEMM uses this tile
 *                   height; 0: chosen per shape.
 * Process-wide, applied at the next launch; not synchronized with launches
 * in flight on other host threads.  Rejects negative max_workgroups and
 * other tile heights (FP4_ERR_ARG).
 */
fp4_status fp4_selftest_set_geometry(int max_workgroups, int gemm_tile_rows);

#ifdef __cplusplus
}
#endif

#endif /* FP4_MI355X_SELFTEST_H */
