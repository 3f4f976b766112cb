/*
 * fp4.h -- C ABI of libfp4_mi355x.so: FP4 (E2M1) block-scaled quantization
 * and the block-scaled GEMMs that consume it, hand-written HIP for gfx950.
 *
 * Method: "Pretraining Large Language Models with NVFP4" (arXiv:2509.25149),
 * App. B (two-level scaling, Eqs. 1-5), §4.2 and App. C (16-point random
 * Hadamard transform on the Wgrad inputs), §4.3 (16x16 2D weight scales),
 * §4.4 (stochastic rounding of gradients), §3 (MXFP4 and NVFP4 formats);
 * the UE5M3 block-scale recipe (arXiv 2609.02846, abstract: unsigned E5M3
 * scales, target T, periodic tensor amax); the 2D-block FP4 recipe
 * (arXiv 2607.24953, abstract: transposition-invariant scales).
 *
 * Conventions shared by every entry point
 *  - Device pointers are HIP device memory of the current device; host
 *    pointers are marked "host".  The caller owns every buffer; the library
 *    allocates nothing and keeps no state between calls.
 *  - bf16 inputs are uint16 bit patterns, row-major with leading dimension
 *    `ld` (elements): the pointer must be 16-byte aligned and ld a multiple
 *    of 8.
 *  - `stream` is a hipStream_t (NULL: the null stream).  Every call only
 *    enqueues work on it; nothing synchronizes with the host, and device
 *    results (amax, s_dec, counters) stay on the device.
 *  - Arguments are validated on the host before any HIP call; a rejected
 *    call returns a nonzero fp4_status, enqueues nothing, and
 *    fp4_last_error() (thread-local) describes why.  A launch failure
 *    returns FP4_ERR_DEVICE.
 *  - Inputs must be finite; rows == 0 or cols == 0 is a valid empty call;
 *    rows and cols of a bf16 input are below 2^31.
 *  - Calls that write the same output buffers on one stream are ordered by
 *    the stream; concurrent calls on different streams must not share
 *    output buffers.
 */
#ifndef FP4_MI355X_H
#define FP4_MI355X_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Every enumeration of this interface is an int: in C++ its underlying type
 * is fixed to int, so any int a caller passes is a value of the type and the
 * argument checks can reject it (without a fixed type, C++ leaves loading a
 * value outside the enumerators' range undefined); in C, an enum is an
 * int-sized integer type already.  The layout is the same in both. */
#ifdef __cplusplus
#define FP4_ENUM_INT : int
#else
#define FP4_ENUM_INT
#endif

/* The FP4 formats' element payload is E2M1 (NVFP4 paper §3: values
 * +-{0,.5,1,1.5,2,3,4,6}), two codes per byte; their block-scale format and
 * block length differ:
 *   FP4_NVFP4  1x16 blocks, E4M3 scale (max 448), fp32 tensor scale  (§3, App. B)
 *   FP4_UE5M3  1x16 blocks, unsigned E5M3 scale (bias 15, all codes finite,
 *              max 122880), fp32 tensor scale with target T          (UE5M3 abstract)
 *   FP4_MXFP4  1x32 blocks, UE8M0 power-of-two scale rounded up, no tensor
 *              scale                                                  (§3, App. B.4)
 * and one 8-bit format, for the attention Q/K projections that the 2D-block
 * FP4 page keeps in MXFP8:
 *   FP4_MXFP8  E4M3 elements (sign in bit 7, max 448), one byte each, in 1x32
 *              blocks with a UE8M0 scale 2^e, e the smallest integer with
 *              448 * 2^e >= amax_B (rounded up like MXFP4's, App. B.4), no
 *              tensor scale; element code = E4M3 RNE of |x * 2^-e|.
 *              Quantize (1D, RNE) and dequantize only: no GEMM takes it. */
typedef enum fp4_format_e FP4_ENUM_INT {
  FP4_NVFP4 = 0, FP4_UE5M3 = 1, FP4_MXFP4 = 2, FP4_MXFP8 = 3
} fp4_format;

/* Element rounding: nearest-even, or stochastic (NVFP4 paper §4.4). */
typedef enum fp4_round_e FP4_ENUM_INT { FP4_RNE = 0, FP4_SR = 1 } fp4_round;

/* Block-scale rounding for NVFP4 / UE5M3: to nearest (NVFP4 paper App. B.2),
 * or up -- the 2D-block FP4 page's truncation-free scaling: the block amax
 * times the encode scale then does not exceed 6, so no element is clipped
 * (up to fp32 rounding of the scale arithmetic).  MXFP4 scales are always
 * rounded up (App. B.4). */
typedef enum fp4_scale_round_e FP4_ENUM_INT { FP4_SCALE_RNE = 0, FP4_SCALE_UP = 1 } fp4_scale_round;

/* 1D blocks along the blocked axis, or 16x16 tiles (NVFP4 paper §4.3). */
typedef enum fp4_block_e FP4_ENUM_INT { FP4_BLOCK_1D = 0, FP4_BLOCK_2D16 = 1 } fp4_block;

/* Where the block scales of a 1D code matrix [R, C] (KB = C / BS blocks per
 * row) are stored.
 *   FP4_SCALES_ROWMAJOR  scale of (row r, block j) at r * KB + j; R * KB bytes.
 *   FP4_SCALES_TILED     at ((r / 256) * KG + j / 8) * 2048 + (r % 256) * 8 + j % 8
 *                        with KG = ceil(KB / 8): 2 KiB atoms, each holding 8
 *                        consecutive blocks of 256 consecutive rows, row by row.
 *                        The buffer is ceil(R / 256) * KG * 2048 bytes and
 *                        16-byte aligned; bytes of rows >= R or blocks >= KB
 *                        are padding, never written and never used.
 * TILED is a storage layout chosen for the GEMM: one 256-row output tile
 * reads the scales of 8 K-blocks as one contiguous 2 KiB run instead of 256
 * scattered pieces.  The scale values are the same in both layouts. */
typedef enum fp4_scale_layout_e FP4_ENUM_INT { FP4_SCALES_ROWMAJOR = 0, FP4_SCALES_TILED = 1 } fp4_scale_layout;

/* ROWWISE: blocks run along cols of X; output is [rows, cols] codes.
 * COLWISE: the matrix quantized is X^T; blocks run along rows of X and the
 * output is the [cols, rows] code matrix of X^T (Wgrad operands, §4.1). */
typedef enum fp4_orient_e FP4_ENUM_INT { FP4_ROWWISE = 0, FP4_COLWISE = 1 } fp4_orient;

/* Span of the global (tensor-level) scale s_enc_G = 6 T / amax, s_dec_G =
 * 1 / s_enc_G (NVFP4 paper App. B.1).  TENSOR: one amax over the whole
 * tensor (a separate pass over x unless given).  ROW: App. B.1 closes by
 * noting the global scale may span a row instead, so no extra round trip
 * through device memory is needed: every row of a ROWWISE 1D code matrix
 * gets its own amax_r = max_c |x[r, c]| (over the rotated row with an RHT),
 * s_enc_r and s_dec_r, read in the same pass that quantizes the row; the
 * GEMM applies s_dec_A[m] s_dec_B[n] to D[m, n].  (A COLWISE row is a
 * column of x spanning every token, which a one-read tile pass cannot see
 * whole before it encodes: COLWISE and 2D16 stay TENSOR.) */
typedef enum fp4_global_scope_e FP4_ENUM_INT { FP4_GLOBAL_TENSOR = 0, FP4_GLOBAL_ROW = 1 } fp4_global_scope;

/* Which events a quantization adds to its fp4_counters (when counters is
 * not NULL).  ALL: every field.  SCALES: the block-scale events only
 * (scale_saturated, scale_underflow, scale_subnormal -- what the UE5M3
 * recipe monitors); the element fields are left unchanged, and the
 * per-element tests, about a quarter of a quantizer's vector work, are
 * skipped.  MX formats have no block-scale events. */
typedef enum fp4_count_level_e FP4_ENUM_INT { FP4_COUNT_ALL = 0, FP4_COUNT_SCALES = 1 } fp4_count_level;

typedef enum fp4_status_e FP4_ENUM_INT {
  FP4_OK = 0,
  FP4_ERR_ARG = 1,          /* null pointer, bad enum, misaligned or bad stride  */
  FP4_ERR_SHAPE = 2,        /* negative size, blocked axis not a block multiple  */
  FP4_ERR_UNSUPPORTED = 3,  /* valid values, combination not defined            */
  FP4_ERR_DEVICE = 4        /* a HIP launch failed                               */
} fp4_status;

/* Quantization events (device memory, accumulated with atomics; the caller
 * zeroes it).  Definitions (block B, y = x * local encode scale):
 *   scale_saturated  the block scale before conversion exceeds the format max
 *   scale_underflow  amax_B > 0 but the block-scale code is 0
 *   scale_subnormal  the block-scale code is a nonzero subnormal
 *   elem_saturated   |y| > 6
 *   elem_underflow   x != 0 but its code is +-0
 * MXFP4 scales are never saturated, underflowed or subnormal. */
typedef struct {
  uint64_t scale_saturated;
  uint64_t scale_underflow;
  uint64_t scale_subnormal;
  uint64_t elem_saturated;
  uint64_t elem_underflow;
} fp4_counters;

/* How to quantize (host struct). */
typedef struct {
  fp4_format format;
  fp4_block block;        /* 2D16: NVFP4/UE5M3, ROWWISE                        */
  fp4_orient orient;
  fp4_round round;        /* SR with 2D16: element (r, c) draws at index
                             r * cols + c, and codes_t is the transposed codes */
  uint64_t seed;          /* SR: Philox4x32-10 key                             */
  uint64_t offset;        /* SR: Philox counter words 2-3 (e.g. a step number) */
  int rht;                /* 1D, NVFP4/UE5M3: rotate every rht_n-element group
                             along the blocked axis by fl32(1/sqrt(N)) D_r H_N
                             first -- rows of a column for COLWISE (the Wgrad
                             operands, App. C), columns of a row for ROWWISE
                             (the Fprop / Dgrad operands, rotated along K by
                             the same signs on both sides, §4.2; §4.2 weighs
                             N = 4, 16, 128 and uses 16)                       */
  uint32_t rht_signs;     /* D_r, bits 0-31: bit i set negates output row i   */
  float target;           /* T in s_enc = 6 T / amax: 448 for NVFP4; 448 or
                             2048 for UE5M3; ignored for MXFP4; finite, > 0    */
  int amax_given;         /* 0: compute the tensor amax into *amax first;
                             1: read *amax (e.g. a stale, periodically
                             refreshed amax); NVFP4/UE5M3 only                 */
  int emit_transpose;     /* 2D16 only: also write the codes of X^T           */
  fp4_scale_layout scale_layout;  /* 1D only: layout of `scales` (TILED: of
                             the output code matrix, [rows, cols] for ROWWISE,
                             [cols, rows] for COLWISE)                         */
  int rht_n;              /* RHT size N: 4, 16, 32, 64 or 128; 0 means 16.
                             Arithmetic: fp32 butterflies with strides 1, 2,
                             ..., N/2, then * fl32(1/sqrt(N)), then the signs;
                             the blocked axis must be a multiple of N          */
  uint32_t rht_signs_hi[3];  /* D_r, bits 32-127 (N > 32); every bit at or
                             above N must be 0                                  */
  fp4_scale_round scale_round;  /* NVFP4/UE5M3 block scales: RNE or UP      */
  fp4_global_scope global_scope;  /* TENSOR, or ROW (NVFP4/UE5M3, 1D ROWWISE,
                             fp4_quantize only): amax and s_dec are then
                             arrays of `rows` floats                          */
  fp4_count_level count_level;    /* events counted into `counters` (the
                             dual quantizer: the same on both sides)         */
} fp4_quant_desc;

/*
 * fp4_amax -- tensor amax (NVFP4 paper App. B.1: amax_X = max |x_i|), the
 * one fp4_quantize computes for `desc` when amax_given = 0.
 *   desc  host; used: orient, rht, rht_n, rht_signs, rht_signs_hi,
 *         global_scope (TENSOR only: fp4_quantize computes per-row amaxes
 *         itself, in the pass that quantizes).  With
 *         rht the amax is taken over the rotated tensor (App. C: the scale
 *         is computed in the rotated space): every rht_n-element group along
 *         the blocked axis -- rows of a column for COLWISE, columns of a row
 *         for ROWWISE -- rotated as fp4_quantize rotates it; that axis must
 *         be a multiple of rht_n.
 *   x     [rows, cols] bf16 (ld), device.
 *   amax  device float, overwritten (0 for an empty tensor).
 */
fp4_status fp4_amax(const fp4_quant_desc* desc /* host */, const uint16_t* x, int64_t rows,
                    int64_t cols, int64_t ld, float* amax, void* stream);

/*
 * fp4_quantize -- quantize a bf16 matrix to E2M1 codes with block scales
 * (NVFP4 paper App. B.1-B.4, Eqs. 1-4; §4.3 2D; §4.4 SR; App. C RHT).
 *
 *   x       [rows, cols] bf16 (ld), device.
 *   codes   device, packed two codes per byte, element 2j in the low nibble
 *           of byte j.  ROWWISE: [rows, cols/2] bytes; COLWISE: [cols, rows/2].
 *           MXFP8: one byte per element, [rows, cols] / [cols, rows].
 *   scales  device, one byte per block.  1D ROWWISE: [rows, cols/BS];
 *           1D COLWISE: [cols, rows/BS]; 2D16: [rows/16, cols/16]
 *           (BS = 16, or 32 for MXFP4 and MXFP8).  1D scales follow desc->scale_layout
 *           (TILED: 16-byte aligned, size as given with fp4_scale_layout).
 *   codes_t device, 2D16 with emit_transpose only: [cols, rows/2] codes of
 *           X^T quantized with the same tile scales (NULL otherwise).
 *   amax    device float.  NVFP4/UE5M3: written (amax_given = 0) or read
 *           (amax_given = 1).  MXFP4, MXFP8: unused, may be NULL.  global_scope
 *           ROW: device float[rows], one amax per row, written or read
 *           likewise (written in the quantizing pass, no separate pass).
 *   s_dec   device float or NULL: receives s_dec_G = 1 / s_enc_G (1 for
 *           MXFP4), the global decode scale the GEMM applies (App. B.3);
 *           global_scope ROW: device float[rows] or NULL, s_dec_r per row.
 *   counters device fp4_counters or NULL (events not counted).
 *   Shapes: the blocked axis (cols for ROWWISE, rows for COLWISE) must be a
 *   multiple of BS; 2D16 needs rows and cols multiples of 16; RHT needs 1D
 *   blocks and the blocked axis a multiple of its size N (rht_n).
 *   SR random bits: element index i in the output code matrix ([R_out,
 *   C_out], i = r * C_out + c) takes 16 bits u of Philox4x32-10(key = seed,
 *   counter = (i >> 3, offset)): output word (i & 7) >> 1, its upper half
 *   for even i, its lower half for odd i.  With lo <= |y| < hi the
 *   neighbouring E2M1 magnitudes and f = (|y| - lo) / (hi - lo), the code
 *   rounds up iff u + floor(65536 f) >= 65536 (the random bits, added to
 *   the first 16 bits of f, carry); |y| >= 6 gives 6.
 */
fp4_status fp4_quantize(const fp4_quant_desc* desc /* host */,
                        const uint16_t* x, int64_t rows, int64_t cols, int64_t ld,
                        uint8_t* codes, uint8_t* scales, uint8_t* codes_t,
                        float* amax, float* s_dec, fp4_counters* counters,
                        void* stream);

/*
 * fp4_quantize_dual -- both 1D quantizations of one bf16 matrix from a
 * single read of it: the ROWWISE code matrix [rows, cols] and the COLWISE
 * code matrix of X^T [cols, rows].  A linear layer needs both of X (Fprop
 * uses the rows, Wgrad the columns) and both of dY (Dgrad, Wgrad)
 * (NVFP4 paper §4.1, Fig. 5); the colwise side may carry the RHT of the
 * Wgrad inputs (§4.2, App. C).  Each output is bit-identical to what
 * fp4_quantize writes with the same descriptor.
 *
 *   row_desc  ROWWISE, 1D; its RHT (along the rows) with rht_n 4 or 16.
 *   col_desc  COLWISE, 1D; its RHT (along the columns) of any size.
 *   Both: global_scope TENSOR (per-row scopes: fp4_quantize).
 *   Both: the same format and the same rounding mode (seed, offset, target,
 *   amax_given, scale_layout, scale_round and the RHT fields are per
 *   side).  When both amaxes are computed here with a 16-point RHT on the
 *   colwise side only, one read of x yields the plain and the rotated amax.
 *   x [rows, cols] bf16 (ld), device; rows and cols multiples of BS.
 *   codes, scales     rowwise outputs, as fp4_quantize with row_desc.
 *   codes_t, scales_t colwise outputs, as fp4_quantize with col_desc.
 *   amax, amax_t      device floats, NVFP4/UE5M3 (MXFP4: unused, may be
 *           NULL): each written (amax_given = 0; in the rotated space of
 *           that side's RHT) or read (amax_given = 1).  They may be the same
 *           buffer only when neither side has an RHT and both sides have the
 *           same amax_given (the amax is then computed once).
 *   s_dec, s_dec_t    device floats or NULL: the two global decode scales.
 *   counters  device fp4_counters or NULL: events of both sides, summed.
 */
fp4_status fp4_quantize_dual(const fp4_quant_desc* row_desc /* host */,
                             const fp4_quant_desc* col_desc /* host */,
                             const uint16_t* x, int64_t rows, int64_t cols, int64_t ld,
                             uint8_t* codes, uint8_t* scales, uint8_t* codes_t, uint8_t* scales_t,
                             float* amax, float* amax_t, float* s_dec, float* s_dec_t,
                             fp4_counters* counters, void* stream);

/*
 * fp4_dequantize -- decode codes and scales: v = fp32(fp32(e2m1 * scale) *
 * s_dec_G) (NVFP4 paper App. B.2-B.3: the decode scales undo the encode
 * scales).  The codes/scales layouts are those fp4_quantize writes for a
 * ROWWISE (or 2D16) [rows, cols] code matrix; 1D scales in scale_layout
 * (2D16 scales are always [rows/16, cols/16]).
 *   s_dec   device float (NVFP4/UE5M3); ignored (may be NULL) for MXFP4.
 *   s_dec_scope  TENSOR: s_dec is one float; ROW (NVFP4/UE5M3, 1D): s_dec
 *           is float[rows], row r decoded with s_dec[r].
 *   out     device, [rows, cols] row-major: fp32 if out_fp32, else bf16
 *           (v rounded to nearest even).
 */
fp4_status fp4_dequantize(fp4_format format, fp4_block block, fp4_scale_layout scale_layout,
                          const uint8_t* codes, const uint8_t* scales, const float* s_dec,
                          fp4_global_scope s_dec_scope, int64_t rows, int64_t cols, void* out,
                          int out_fp32, void* stream);

/*
 * fp4_rht16 -- the random Hadamard transform alone (NVFP4 paper §4.2,
 * App. C): y = fl32(1/sqrt(N)) D_r H_N v for every N-element group v along
 * the blocked axis of `desc` -- N consecutive rows of a column (COLWISE) or
 * N consecutive columns of a row (ROWWISE); N = rht_n (0 means 16, the
 * 16-point transform: scale exactly 1/4).  fp32 arithmetic as a
 * Walsh-Hadamard butterfly network with strides 1, 2, ..., N/2 (each
 * butterfly (a, b) -> (a + b, a - b)), then the scale, then the sign flips
 * (bit i of rht_signs / rht_signs_hi negates entry i of each group); these
 * are the values fp4_quantize with rht = 1 quantizes.
 *   desc  host; used: orient, rht_n, rht_signs, rht_signs_hi (rht ignored).
 *   x [rows, cols] bf16 (ld), device; the rotated axis a multiple of N.
 *   y [rows, cols] fp32 row-major (leading dimension cols), device,
 *     16-byte aligned.
 */
fp4_status fp4_rht16(const fp4_quant_desc* desc /* host */, const uint16_t* x, int64_t rows,
                     int64_t cols, int64_t ld, float* y, void* stream);

/* One GEMM operand: a [rows, K] code matrix, K-major (host struct of device
 * pointers).  With scale_layout ROWMAJOR the scale of (row r, K-block j) is
 *   scales[(r / scale_row_group) * scale_stride_row + j * scale_stride_kblk]
 * so 1D scales are (row_group 1, stride_row K/BS, stride_kblk 1); 2D16
 * scales of W are (16, K/16, 1); the 2D16 scales of W used for the codes_t
 * matrix W^T are (16, 1, rows_of_W/16) -- the same bytes (§4.3: the tile
 * scale is replicated per 1x16 block).  With scale_layout TILED the scales
 * are the TILED layout of the [rows, K] code matrix (KB = K / BS); the
 * strides are ignored, scale_row_group must be 1 and `scales` 16-byte
 * aligned. */
typedef struct {
  fp4_format format;
  const uint8_t* codes;       /* device, 16-byte aligned; ld_codes bytes per row,
                                 ld_codes >= K/2 and a multiple of 8 (16 for MXFP4) */
  int64_t ld_codes;
  const uint8_t* scales;      /* device */
  int64_t scale_stride_row;
  int64_t scale_stride_kblk;
  int32_t scale_row_group;    /* 1 or 16 */
  const float* s_dec;         /* device s_dec_G; NULL means 1 (MXFP4 ignores it) */
  fp4_scale_layout scale_layout;
  fp4_global_scope s_dec_scope;  /* TENSOR: s_dec is one float; ROW (NVFP4/UE5M3):
                                 s_dec[rows], one per operand row (non-NULL) */
} fp4_operand;

/* Element type of a GEMM output (NVFP4 paper §4.1: the GEMMs take FP4
 * inputs and write BF16 or FP32). */
typedef enum fp4_out_type_e FP4_ENUM_INT { FP4_OUT_F32 = 0, FP4_OUT_BF16 = 1 } fp4_out_type;

/*
 * fp4_gemm -- D[M, N] (+)= s_dec_A * s_dec_B * sum_k a[m, k] * b[n, k]
 * (s_dec_A[m] and s_dec_B[n] for operands with per-row global scales),
 * a = e2m1 * scale of A [M, K], b likewise of B [N, K] ("TN": both K-major).
 * This is the block-scaled product of NVFP4 paper App. B.3 (per-block
 * partial products scaled by both local decode scales, fp32 accumulation,
 * global decode scales applied to the output) used for Fprop, Dgrad and
 * Wgrad (§4.1, Fig. 5).  A and B must have the same format; K must be a
 * multiple of the format's block length.
 *   D  device, row-major with leading dimension ldd >= N (in elements of
 *      d_type): fp32 (FP4_OUT_F32), or bf16 bits (FP4_OUT_BF16: every value
 *      is formed in fp32 as for an fp32 D -- with accumulate, the old bf16
 *      value widened and added in fp32 -- then rounded once to nearest even).
 *   accumulate  0: D = result; 1: D += result (e.g. Wgrad accumulation).
 * Accuracy (fp32 D): |D - exact| <= 1e-5 * s_dec_A * s_dec_B * sum_k |a b|
 * per element; a bf16 D is that fp32 value rounded to bf16.
 * K == 0 writes zeros (or leaves D unchanged when accumulating).
 */
fp4_status fp4_gemm(const fp4_operand* A /* host */, const fp4_operand* B /* host */,
                    int64_t M, int64_t N, int64_t K, void* D, fp4_out_type d_type,
                    int64_t ldd, int accumulate, void* stream);

/* Static description of a status code. */
const char* fp4_status_string(fp4_status status);

/* Thread-local detail of the last rejected or failed call on this thread
 * ("" if none). */
const char* fp4_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* FP4_MI355X_H */
