// C ABI of libfp4_mi355x.so (declared in include/fp4.h): host-side argument
// validation, then kernel launches on the caller's stream.  Validation
// touches no HIP API, so rejected calls work without a GPU.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <string>

#include "../../include/fp4.h"
#include "../../include/fp4_selftest.h"
#include "fp4_internal.hpp"

#define FP4_EXPORT extern "C" __attribute__((visibility("default")))

namespace {

thread_local std::string g_last_error;

fp4_status fail(fp4_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

fp4_status ok() {
  g_last_error.clear();
  return FP4_OK;
}

fp4_status device_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(FP4_ERR_DEVICE, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// MX formats: 1x32 blocks of power-of-two scales and no tensor scale.
bool is_mx(fp4_format f) { return f == FP4_MXFP4 || f == FP4_MXFP8; }

int block_len(fp4_format f) { return is_mx(f) ? 32 : 16; }

bool valid_format(int f) {
  return f == FP4_NVFP4 || f == FP4_UE5M3 || f == FP4_MXFP4 || f == FP4_MXFP8;
}

int rht_size(const fp4_quant_desc* d) { return d->rht_n ? d->rht_n : 16; }

// RHT size and sign mask of a descriptor (checked only when rht is on).
fp4_status check_rht(const fp4_quant_desc* d, const char* side) {
  if (!d->rht) return FP4_OK;
  const int n = rht_size(d);
  if (n != 4 && n != 16 && n != 32 && n != 64 && n != 128)
    return fail(FP4_ERR_ARG, "%s: rht_n=%d must be 4, 16, 32, 64 or 128", side, d->rht_n);
  const uint32_t w[4] = {d->rht_signs, d->rht_signs_hi[0], d->rht_signs_hi[1], d->rht_signs_hi[2]};
  for (int i = 0; i < 4; ++i) {
    const int lo = 32 * i;                          // first bit of word i
    const uint32_t allowed = n >= lo + 32 ? 0xFFFFFFFFu : n <= lo ? 0u : ((1u << (n - lo)) - 1u);
    if (w[i] & ~allowed) return fail(FP4_ERR_ARG, "%s: rht sign bits at or above N=%d", side, n);
  }
  return FP4_OK;
}

void copy_signs(const fp4_quant_desc* d, uint32_t (&out)[4]) {
  out[0] = d->rht_signs;
  for (int i = 0; i < 3; ++i) out[i + 1] = d->rht_signs_hi[i];
}

fp4_status check_bf16_input(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld) {
  if (rows < 0 || cols < 0) return fail(FP4_ERR_SHAPE, "negative size rows=%lld cols=%lld",
                                        (long long)rows, (long long)cols);
  if (rows >= (int64_t(1) << 31) || cols >= (int64_t(1) << 31))
    return fail(FP4_ERR_SHAPE, "rows=%lld and cols=%lld must be below 2^31", (long long)rows,
                (long long)cols);
  if (ld < cols) return fail(FP4_ERR_ARG, "ld=%lld < cols=%lld", (long long)ld, (long long)cols);
  if (rows > 0 && cols > 0) {
    if (!x) return fail(FP4_ERR_ARG, "x is null");
    if (!aligned16(x)) return fail(FP4_ERR_ARG, "x must be 16-byte aligned");
    if (ld % 8) return fail(FP4_ERR_ARG, "ld=%lld must be a multiple of 8", (long long)ld);
    if (cols % 8) return fail(FP4_ERR_SHAPE, "cols=%lld must be a multiple of 8", (long long)cols);
  }
  return ok();
}

}  // namespace

FP4_EXPORT const char* fp4_status_string(fp4_status s) {
  switch (s) {
    case FP4_OK: return "ok";
    case FP4_ERR_ARG: return "invalid argument";
    case FP4_ERR_SHAPE: return "invalid shape";
    case FP4_ERR_UNSUPPORTED: return "unsupported combination";
    case FP4_ERR_DEVICE: return "device error";
  }
  return "unknown status";
}

FP4_EXPORT const char* fp4_last_error(void) { return g_last_error.c_str(); }

FP4_EXPORT fp4_status fp4_amax(const fp4_quant_desc* d, const uint16_t* x, int64_t rows,
                               int64_t cols, int64_t ld, float* amax, void* stream) {
  if (!d) return fail(FP4_ERR_ARG, "desc is null");
  if (d->orient != FP4_ROWWISE && d->orient != FP4_COLWISE)
    return fail(FP4_ERR_ARG, "bad orient %d", (int)d->orient);
  fp4_status st = check_bf16_input(x, rows, cols, ld);
  if (st) return st;
  if (!amax) return fail(FP4_ERR_ARG, "amax is null");
  if (d->global_scope != FP4_GLOBAL_TENSOR)
    return fail(FP4_ERR_UNSUPPORTED, "fp4_amax computes the tensor amax only (per-row amaxes "
                                     "come from fp4_quantize with global_scope ROW)");
  st = check_rht(d, "desc");
  if (st) return st;
  const bool along_rows = d->orient == FP4_ROWWISE;
  if (d->rht && (along_rows ? cols : rows) % rht_size(d))
    return fail(FP4_ERR_SHAPE, "the rotated axis (%s=%lld) must be a multiple of rht_n=%d",
                along_rows ? "cols" : "rows", (long long)(along_rows ? cols : rows), rht_size(d));
  uint32_t s4[4];
  copy_signs(d, s4);
  return device_status(fp4lib::launch_amax(x, rows, cols, ld, d->rht, rht_size(d), s4, amax,
                                           static_cast<hipStream_t>(stream), nullptr, along_rows),
                       "fp4_amax launch");
}

FP4_EXPORT fp4_status fp4_quantize(const fp4_quant_desc* d, const uint16_t* x, int64_t rows,
                                   int64_t cols, int64_t ld, uint8_t* codes, uint8_t* scales,
                                   uint8_t* codes_t, float* amax, float* s_dec,
                                   fp4_counters* counters, void* stream) {
  if (!d) return fail(FP4_ERR_ARG, "desc is null");
  if (!valid_format(d->format)) return fail(FP4_ERR_ARG, "bad format %d", (int)d->format);
  if (d->block != FP4_BLOCK_1D && d->block != FP4_BLOCK_2D16)
    return fail(FP4_ERR_ARG, "bad block %d", (int)d->block);
  if (d->orient != FP4_ROWWISE && d->orient != FP4_COLWISE)
    return fail(FP4_ERR_ARG, "bad orient %d", (int)d->orient);
  if (d->round != FP4_RNE && d->round != FP4_SR) return fail(FP4_ERR_ARG, "bad round %d", (int)d->round);
  fp4_status st = check_bf16_input(x, rows, cols, ld);
  if (st) return st;
  const bool two_level = !is_mx(d->format);
  const bool mx8 = d->format == FP4_MXFP8;
  const bool is2d = d->block == FP4_BLOCK_2D16;
  const int bs = block_len(d->format);
  if (is2d && !two_level) return fail(FP4_ERR_UNSUPPORTED, "2D16 blocks need NVFP4 or UE5M3");
  if (mx8 && d->round != FP4_RNE) return fail(FP4_ERR_UNSUPPORTED, "MXFP8 rounds to nearest even");
  if (is2d && d->orient != FP4_ROWWISE) return fail(FP4_ERR_UNSUPPORTED, "2D16 blocks are ROWWISE only");
  if (d->scale_round != FP4_SCALE_RNE && d->scale_round != FP4_SCALE_UP)
    return fail(FP4_ERR_ARG, "bad scale_round %d", (int)d->scale_round);
  if (d->rht && is2d) return fail(FP4_ERR_UNSUPPORTED, "RHT needs 1D blocks");
  if (d->rht && !two_level) return fail(FP4_ERR_UNSUPPORTED, "RHT needs NVFP4 or UE5M3");
  st = check_rht(d, "desc");
  if (st) return st;
  if (d->amax_given && !two_level) return fail(FP4_ERR_UNSUPPORTED, "MX formats have no tensor amax");
  if (d->global_scope != FP4_GLOBAL_TENSOR && d->global_scope != FP4_GLOBAL_ROW)
    return fail(FP4_ERR_ARG, "bad global_scope %d", (int)d->global_scope);
  if (d->count_level != FP4_COUNT_ALL && d->count_level != FP4_COUNT_SCALES)
    return fail(FP4_ERR_ARG, "bad count_level %d", (int)d->count_level);
  const bool row_scope = d->global_scope == FP4_GLOBAL_ROW;
  if (row_scope && (!two_level || is2d || d->orient != FP4_ROWWISE))
    return fail(FP4_ERR_UNSUPPORTED, "global_scope ROW needs NVFP4 or UE5M3, 1D, ROWWISE");
  if (!is2d && d->emit_transpose) return fail(FP4_ERR_UNSUPPORTED, "emit_transpose needs 2D16");
  if (d->scale_layout != FP4_SCALES_ROWMAJOR && d->scale_layout != FP4_SCALES_TILED)
    return fail(FP4_ERR_ARG, "bad scale_layout %d", (int)d->scale_layout);
  const bool tiled = d->scale_layout == FP4_SCALES_TILED;
  if (tiled && is2d) return fail(FP4_ERR_UNSUPPORTED, "TILED scales are for 1D blocks");
  if (two_level && !(std::isfinite(d->target) && d->target > 0.0f))
    return fail(FP4_ERR_ARG, "target must be finite and > 0");
  if (is2d) {
    if (rows % 16 || cols % 16)
      return fail(FP4_ERR_SHAPE, "2D16 needs rows, cols multiples of 16 (%lld x %lld)",
                  (long long)rows, (long long)cols);
  } else if (d->orient == FP4_ROWWISE) {
    if (cols % bs) return fail(FP4_ERR_SHAPE, "cols=%lld must be a multiple of %d", (long long)cols, bs);
    if (d->rht && cols % rht_size(d))
      return fail(FP4_ERR_SHAPE, "cols=%lld must be a multiple of rht_n=%d", (long long)cols,
                  rht_size(d));
  } else {
    if (rows % bs) return fail(FP4_ERR_SHAPE, "rows=%lld must be a multiple of %d", (long long)rows, bs);
    if (d->rht && rows % rht_size(d))
      return fail(FP4_ERR_SHAPE, "rows=%lld must be a multiple of rht_n=%d", (long long)rows,
                  rht_size(d));
  }
  const bool empty = rows == 0 || cols == 0;
  if (!empty) {
    if (!codes || !scales) return fail(FP4_ERR_ARG, "codes/scales are null");
    if (!aligned16(codes)) return fail(FP4_ERR_ARG, "codes must be 16-byte aligned");
    if (tiled && !aligned16(scales)) return fail(FP4_ERR_ARG, "TILED scales must be 16-byte aligned");
    if (d->emit_transpose && (!codes_t || !aligned16(codes_t)))
      return fail(FP4_ERR_ARG, "codes_t must be non-null and 16-byte aligned");
  }
  if (two_level && !amax) return fail(FP4_ERR_ARG, "amax is null");

  hipStream_t s = static_cast<hipStream_t>(stream);
  if (two_level && !d->amax_given && !row_scope) {
    uint32_t s4[4];
    copy_signs(d, s4);
    hipError_t e = fp4lib::launch_amax(x, rows, cols, ld, d->rht, rht_size(d), s4, amax, s,
                                       nullptr, d->orient == FP4_ROWWISE);
    if (e != hipSuccess) return device_status(e, "fp4_quantize amax launch");
  }
  fp4lib::QuantArgs a{};
  a.x = x;
  a.rows = rows;
  a.cols = cols;
  a.ld = ld;
  a.codes = codes;
  a.scales = scales;
  a.codes_t = codes_t;
  a.amax = amax;
  a.s_dec = s_dec;
  a.counters = counters;
  a.target = d->target;
  a.seed = d->seed;
  a.offset = d->offset;
  copy_signs(d, a.rht_signs);
  a.rht_n = rht_size(d);
  a.scale_up = two_level && d->scale_round == FP4_SCALE_UP;
  a.format = d->format;
  a.round = d->round;
  a.rht = d->rht;
  a.emit_transpose = d->emit_transpose;
  a.tiled = tiled ? 1 : 0;
  a.amax_given = d->amax_given ? 1 : 0;
  a.count_elems = d->count_level == FP4_COUNT_ALL ? 1 : 0;
  hipError_t e;
  if (mx8) e = fp4lib::launch_quant_mx8(a, d->orient == FP4_COLWISE, s);
  else if (row_scope) e = fp4lib::launch_quant_row_scoped(a, s);
  else if (is2d) e = fp4lib::launch_quant_2d(a, s);
  else if (d->orient == FP4_ROWWISE) e = fp4lib::launch_quant_row(a, s);
  else e = fp4lib::launch_quant_col(a, s);
  return device_status(e, "fp4_quantize launch");
}

FP4_EXPORT fp4_status fp4_quantize_dual(const fp4_quant_desc* rd, const fp4_quant_desc* cd,
                                        const uint16_t* x, int64_t rows, int64_t cols, int64_t ld,
                                        uint8_t* codes, uint8_t* scales, uint8_t* codes_t,
                                        uint8_t* scales_t, float* amax, float* amax_t,
                                        float* s_dec, float* s_dec_t, fp4_counters* counters,
                                        void* stream) {
  if (!rd || !cd) return fail(FP4_ERR_ARG, "desc is null");
  const fp4_quant_desc* ds[2] = {rd, cd};
  for (int i = 0; i < 2; ++i) {
    const fp4_quant_desc* d = ds[i];
    const char* side = i ? "colwise" : "rowwise";
    if (!valid_format(d->format)) return fail(FP4_ERR_ARG, "%s: bad format %d", side, (int)d->format);
    if (d->format == FP4_MXFP8)
      return fail(FP4_ERR_UNSUPPORTED, "%s: dual quantization takes the FP4 formats", side);
    if (d->block != FP4_BLOCK_1D && d->block != FP4_BLOCK_2D16)
      return fail(FP4_ERR_ARG, "%s: bad block %d", side, (int)d->block);
    if (d->orient != FP4_ROWWISE && d->orient != FP4_COLWISE)
      return fail(FP4_ERR_ARG, "%s: bad orient %d", side, (int)d->orient);
    if (d->round != FP4_RNE && d->round != FP4_SR)
      return fail(FP4_ERR_ARG, "%s: bad round %d", side, (int)d->round);
    if (d->scale_layout != FP4_SCALES_ROWMAJOR && d->scale_layout != FP4_SCALES_TILED)
      return fail(FP4_ERR_ARG, "%s: bad scale_layout %d", side, (int)d->scale_layout);
    if (d->block != FP4_BLOCK_1D) return fail(FP4_ERR_UNSUPPORTED, "%s: dual quantization is 1D", side);
    if (d->emit_transpose) return fail(FP4_ERR_UNSUPPORTED, "%s: emit_transpose needs 2D16", side);
    if (d->format != FP4_MXFP4 && !(std::isfinite(d->target) && d->target > 0.0f))
      return fail(FP4_ERR_ARG, "%s: target must be finite and > 0", side);
    if (d->amax_given && d->format == FP4_MXFP4)
      return fail(FP4_ERR_UNSUPPORTED, "%s: MXFP4 has no tensor amax", side);
    if (d->scale_round != FP4_SCALE_RNE && d->scale_round != FP4_SCALE_UP)
      return fail(FP4_ERR_ARG, "%s: bad scale_round %d", side, (int)d->scale_round);
    if (d->global_scope != FP4_GLOBAL_TENSOR)
      return fail(FP4_ERR_UNSUPPORTED, "%s: dual quantization has tensor-scope global scales "
                                       "(per-row scales: fp4_quantize ROWWISE)", side);
    if (d->count_level != FP4_COUNT_ALL && d->count_level != FP4_COUNT_SCALES)
      return fail(FP4_ERR_ARG, "%s: bad count_level %d", side, (int)d->count_level);
  }
  if (rd->count_level != cd->count_level)
    return fail(FP4_ERR_UNSUPPORTED, "the two descs count different events");
  if (rd->orient != FP4_ROWWISE || cd->orient != FP4_COLWISE)
    return fail(FP4_ERR_UNSUPPORTED, "descs must be ROWWISE then COLWISE");
  if (rd->format != cd->format) return fail(FP4_ERR_UNSUPPORTED, "the two formats differ");
  if (rd->round != cd->round) return fail(FP4_ERR_UNSUPPORTED, "the two rounding modes differ");
  if ((rd->rht || cd->rht) && cd->format == FP4_MXFP4)
    return fail(FP4_ERR_UNSUPPORTED, "RHT needs NVFP4 or UE5M3");
  if (rd->rht && rht_size(rd) != 4 && rht_size(rd) != 16)
    return fail(FP4_ERR_UNSUPPORTED, "rowwise RHT of the dual quantizer: rht_n must be 4 or 16");
  fp4_status st0 = check_rht(rd, "rowwise");
  if (st0) return st0;
  st0 = check_rht(cd, "colwise");
  if (st0) return st0;
  fp4_status st = check_bf16_input(x, rows, cols, ld);
  if (st) return st;
  const int bs = block_len(rd->format);
  if (cols % bs || rows % bs)
    return fail(FP4_ERR_SHAPE, "rows=%lld and cols=%lld must be multiples of %d", (long long)rows,
                (long long)cols, bs);
  if (cd->rht && rows % rht_size(cd))
    return fail(FP4_ERR_SHAPE, "rows=%lld must be a multiple of rht_n=%d", (long long)rows,
                rht_size(cd));
  if (rd->rht && cols % rht_size(rd))
    return fail(FP4_ERR_SHAPE, "cols=%lld must be a multiple of rht_n=%d", (long long)cols,
                rht_size(rd));
  const bool two_level = rd->format != FP4_MXFP4;
  const bool empty = rows == 0 || cols == 0;
  if (!empty) {
    if (!codes || !scales || !codes_t || !scales_t) return fail(FP4_ERR_ARG, "codes/scales are null");
    if (!aligned16(codes) || !aligned16(codes_t))
      return fail(FP4_ERR_ARG, "codes and codes_t must be 16-byte aligned");
    if ((rd->scale_layout == FP4_SCALES_TILED && !aligned16(scales)) ||
        (cd->scale_layout == FP4_SCALES_TILED && !aligned16(scales_t)))
      return fail(FP4_ERR_ARG, "TILED scales must be 16-byte aligned");
  }
  if (two_level) {
    if (!amax || !amax_t) return fail(FP4_ERR_ARG, "amax/amax_t is null");
    if (amax == amax_t && (rd->amax_given != cd->amax_given || cd->rht || rd->rht))
      return fail(FP4_ERR_ARG, "amax and amax_t may share a buffer only without RHT and with "
                               "the same amax_given");
  }

  hipStream_t s = static_cast<hipStream_t>(stream);
  // both amaxes wanted with the 16-point RHT on the colwise side: one read
  const bool fused = two_level && !rd->amax_given && !cd->amax_given && cd->rht && !rd->rht &&
                     rht_size(cd) == 16 && amax != amax_t;
  if (fused) {
    uint32_t s4[4];
    copy_signs(cd, s4);
    hipError_t e = fp4lib::launch_amax(x, rows, cols, ld, 1, 16, s4, amax_t, s, amax);
    if (e != hipSuccess) return device_status(e, "fp4_quantize_dual amax launch");
  }
  if (two_level && !rd->amax_given && !fused) {
    uint32_t s4[4];
    copy_signs(rd, s4);
    hipError_t e = fp4lib::launch_amax(x, rows, cols, ld, rd->rht, rht_size(rd), s4, amax, s,
                                       nullptr, true);
    if (e != hipSuccess) return device_status(e, "fp4_quantize_dual amax launch");
  }
  if (two_level && !cd->amax_given && !fused && !(amax_t == amax && !rd->amax_given)) {
    uint32_t s4[4];
    copy_signs(cd, s4);
    hipError_t e = fp4lib::launch_amax(x, rows, cols, ld, cd->rht, rht_size(cd), s4, amax_t, s);
    if (e != hipSuccess) return device_status(e, "fp4_quantize_dual amax launch");
  }
  fp4lib::QuantArgs a[2]{};
  uint8_t* cs[2] = {codes, codes_t};
  uint8_t* ss[2] = {scales, scales_t};
  float* am[2] = {amax, amax_t};
  float* sd[2] = {s_dec, s_dec_t};
  for (int i = 0; i < 2; ++i) {
    a[i].x = x;
    a[i].rows = rows;
    a[i].cols = cols;
    a[i].ld = ld;
    a[i].codes = cs[i];
    a[i].scales = ss[i];
    a[i].amax = am[i];
    a[i].s_dec = sd[i];
    a[i].counters = counters;
    a[i].target = ds[i]->target;
    a[i].seed = ds[i]->seed;
    a[i].offset = ds[i]->offset;
    copy_signs(ds[i], a[i].rht_signs);
    a[i].rht_n = rht_size(ds[i]);
    a[i].count_elems = ds[i]->count_level == FP4_COUNT_ALL ? 1 : 0;
    a[i].scale_up = ds[i]->format != FP4_MXFP4 && ds[i]->scale_round == FP4_SCALE_UP;
    a[i].format = ds[i]->format;
    a[i].round = ds[i]->round;
    a[i].rht = ds[i]->rht;
    a[i].tiled = ds[i]->scale_layout == FP4_SCALES_TILED ? 1 : 0;
  }
  return device_status(fp4lib::launch_quant_dual(a[0], a[1], s), "fp4_quantize_dual launch");
}

FP4_EXPORT fp4_status fp4_dequantize(fp4_format format, fp4_block block,
                                     fp4_scale_layout scale_layout, const uint8_t* codes,
                                     const uint8_t* scales, const float* s_dec,
                                     fp4_global_scope s_dec_scope, int64_t rows, int64_t cols,
                                     void* out, int out_fp32, void* stream) {
  if (!valid_format(format)) return fail(FP4_ERR_ARG, "bad format %d", (int)format);
  if (block != FP4_BLOCK_1D && block != FP4_BLOCK_2D16) return fail(FP4_ERR_ARG, "bad block %d", (int)block);
  if (scale_layout != FP4_SCALES_ROWMAJOR && scale_layout != FP4_SCALES_TILED)
    return fail(FP4_ERR_ARG, "bad scale_layout %d", (int)scale_layout);
  const bool tiled = scale_layout == FP4_SCALES_TILED;
  if (tiled && block == FP4_BLOCK_2D16) return fail(FP4_ERR_UNSUPPORTED, "TILED scales are for 1D blocks");
  if (block == FP4_BLOCK_2D16 && is_mx(format))
    return fail(FP4_ERR_UNSUPPORTED, "2D16 blocks need NVFP4 or UE5M3");
  if (s_dec_scope != FP4_GLOBAL_TENSOR && s_dec_scope != FP4_GLOBAL_ROW)
    return fail(FP4_ERR_ARG, "bad s_dec_scope %d", (int)s_dec_scope);
  const bool s_dec_rows = s_dec_scope == FP4_GLOBAL_ROW;
  if (s_dec_rows && (is_mx(format) || block != FP4_BLOCK_1D))
    return fail(FP4_ERR_UNSUPPORTED, "per-row s_dec needs NVFP4 or UE5M3 and 1D blocks");
  if (rows < 0 || cols < 0) return fail(FP4_ERR_SHAPE, "negative size");
  const int bs = block_len(format);
  if (cols % bs) return fail(FP4_ERR_SHAPE, "cols=%lld must be a multiple of %d", (long long)cols, bs);
  if (block == FP4_BLOCK_2D16 && rows % 16) return fail(FP4_ERR_SHAPE, "2D16 needs rows %% 16 == 0");
  if (rows > 0 && cols > 0) {
    if (!codes || !scales || !out) return fail(FP4_ERR_ARG, "null pointer");
    if (!aligned16(codes) || !aligned16(out)) return fail(FP4_ERR_ARG, "codes/out must be 16-byte aligned");
    if (tiled && !aligned16(scales)) return fail(FP4_ERR_ARG, "TILED scales must be 16-byte aligned");
    if (!is_mx(format) && !s_dec) return fail(FP4_ERR_ARG, "s_dec is null");
  }
  if (rows == 0 || cols == 0) return ok();
  if (format == FP4_MXFP8)
    return device_status(fp4lib::launch_dequant_mx8(tiled, codes, scales, rows, cols, out,
                                                    out_fp32, static_cast<hipStream_t>(stream)),
                         "fp4_dequantize launch");
  return device_status(fp4lib::launch_dequant(format, block == FP4_BLOCK_2D16, tiled, codes, scales,
                                              s_dec, s_dec_rows, rows, cols, out, out_fp32,
                                              static_cast<hipStream_t>(stream)),
                       "fp4_dequantize launch");
}

FP4_EXPORT fp4_status fp4_rht16(const fp4_quant_desc* d, const uint16_t* x, int64_t rows,
                                int64_t cols, int64_t ld, float* y, void* stream) {
  if (!d) return fail(FP4_ERR_ARG, "desc is null");
  if (d->orient != FP4_ROWWISE && d->orient != FP4_COLWISE)
    return fail(FP4_ERR_ARG, "bad orient %d", (int)d->orient);
  fp4_status st = check_bf16_input(x, rows, cols, ld);
  if (st) return st;
  fp4_quant_desc on = *d;
  on.rht = 1;                                  // the transform itself is always applied
  st = check_rht(&on, "desc");
  if (st) return st;
  const bool along_rows = d->orient == FP4_ROWWISE;
  if ((along_rows ? cols : rows) % rht_size(d))
    return fail(FP4_ERR_SHAPE, "the rotated axis (%s=%lld) must be a multiple of rht_n=%d",
                along_rows ? "cols" : "rows", (long long)(along_rows ? cols : rows), rht_size(d));
  if (rows > 0 && cols > 0 && (!y || (reinterpret_cast<uintptr_t>(y) & 15u)))
    return fail(FP4_ERR_ARG, "y must be non-null and 16-byte aligned");
  if (rows == 0 || cols == 0) return ok();
  uint32_t s4[4];
  copy_signs(d, s4);
  return device_status(fp4lib::launch_rht(x, rows, cols, ld, rht_size(d), s4, along_rows, y,
                                          static_cast<hipStream_t>(stream)),
                       "fp4_rht16 launch");
}

FP4_EXPORT fp4_status fp4_gemm(const fp4_operand* A, const fp4_operand* B, int64_t M, int64_t N,
                               int64_t K, void* D, fp4_out_type d_type, int64_t ldd,
                               int accumulate, void* stream) {
  if (!A || !B) return fail(FP4_ERR_ARG, "operand descriptor is null");
  if (!valid_format(A->format) || !valid_format(B->format)) return fail(FP4_ERR_ARG, "bad format");
  if (A->format != B->format) return fail(FP4_ERR_UNSUPPORTED, "A and B formats differ");
  if (A->format == FP4_MXFP8) return fail(FP4_ERR_UNSUPPORTED, "no GEMM takes MXFP8 operands");
  if (M < 0 || N < 0 || K < 0) return fail(FP4_ERR_SHAPE, "negative size");
  const int bs = block_len(A->format);
  if (K % bs) return fail(FP4_ERR_SHAPE, "K=%lld must be a multiple of %d", (long long)K, bs);
  if (ldd < N) return fail(FP4_ERR_ARG, "ldd=%lld < N=%lld", (long long)ldd, (long long)N);
  if (d_type != FP4_OUT_F32 && d_type != FP4_OUT_BF16)
    return fail(FP4_ERR_ARG, "bad d_type %d", (int)d_type);
  const fp4_operand* ops[2] = {A, B};
  for (int i = 0; i < 2; ++i) {
    const fp4_operand* o = ops[i];
    if (o->scale_row_group != 1 && o->scale_row_group != 16)
      return fail(FP4_ERR_ARG, "scale_row_group must be 1 or 16");
    if (o->scale_layout != FP4_SCALES_ROWMAJOR && o->scale_layout != FP4_SCALES_TILED)
      return fail(FP4_ERR_ARG, "operand %c: bad scale_layout %d", "AB"[i], (int)o->scale_layout);
    if (o->scale_layout == FP4_SCALES_TILED && o->scale_row_group != 1)
      return fail(FP4_ERR_UNSUPPORTED, "operand %c: TILED scales need scale_row_group 1", "AB"[i]);
    if (o->scale_row_group == 16 && A->format == FP4_MXFP4)
      return fail(FP4_ERR_UNSUPPORTED, "2D16 scales need NVFP4 or UE5M3");
    if (o->s_dec_scope != FP4_GLOBAL_TENSOR && o->s_dec_scope != FP4_GLOBAL_ROW)
      return fail(FP4_ERR_ARG, "operand %c: bad s_dec_scope %d", "AB"[i], (int)o->s_dec_scope);
    if (o->s_dec_scope == FP4_GLOBAL_ROW && (A->format == FP4_MXFP4 || !o->s_dec))
      return fail(FP4_ERR_UNSUPPORTED, "operand %c: per-row s_dec needs NVFP4 or UE5M3 and a "
                                       "non-null s_dec", "AB"[i]);
    if (M > 0 && N > 0 && K > 0) {
      if (!o->codes || !o->scales) return fail(FP4_ERR_ARG, "operand %c has a null pointer", "AB"[i]);
      if (o->ld_codes < K / 2) return fail(FP4_ERR_ARG, "operand %c ld_codes < K/2", "AB"[i]);
      const int ld_align = A->format == FP4_MXFP4 ? 16 : 8;
      if (!aligned16(o->codes) || o->ld_codes % ld_align)
        return fail(FP4_ERR_ARG, "operand %c codes must be 16-byte aligned with ld_codes %% %d == 0",
                    "AB"[i], ld_align);
      if (o->scale_stride_row < 0 || o->scale_stride_kblk < 0)
        return fail(FP4_ERR_ARG, "negative scale stride");
      if (o->scale_layout == FP4_SCALES_TILED && !aligned16(o->scales))
        return fail(FP4_ERR_ARG, "operand %c: TILED scales must be 16-byte aligned", "AB"[i]);
    }
  }
  if (M > 0 && N > 0 && !D) return fail(FP4_ERR_ARG, "D is null");
  if (M == 0 || N == 0) return ok();
  fp4lib::GemmOperand a{A->codes, A->ld_codes, A->scales, A->scale_stride_row,
                        A->scale_stride_kblk, A->scale_row_group, A->s_dec,
                        A->scale_layout == FP4_SCALES_TILED, A->s_dec_scope == FP4_GLOBAL_ROW};
  fp4lib::GemmOperand b{B->codes, B->ld_codes, B->scales, B->scale_stride_row,
                        B->scale_stride_kblk, B->scale_row_group, B->s_dec,
                        B->scale_layout == FP4_SCALES_TILED, B->s_dec_scope == FP4_GLOBAL_ROW};
  return device_status(fp4lib::launch_gemm(A->format, a, b, M, N, K, D, d_type == FP4_OUT_BF16,
                                           ldd, accumulate,
                                           static_cast<hipStream_t>(stream)),
                       "fp4_gemm launch");
}

FP4_EXPORT fp4_status fp4_selftest_set_geometry(int max_workgroups, int gemm_tile_rows) {
  if (max_workgroups < 0) return fail(FP4_ERR_ARG, "max_workgroups must be >= 0");
  if (gemm_tile_rows != 0 && gemm_tile_rows != 192 && gemm_tile_rows != 256)
    return fail(FP4_ERR_ARG, "gemm_tile_rows must be 0, 192 or 256");
  fp4lib::set_launch_geometry(max_workgroups, gemm_tile_rows);
  return ok();
}

FP4_EXPORT fp4_status fp4_selftest_sweep(int kind, const uint32_t* thresholds, int n,
                                         uint64_t* result, void* stream) {
  static const int kLen[5] = {7, 126, 255, 7, 126};
  if (kind < FP4_SWEEP_E2M1_RNE || kind > FP4_SWEEP_E4M3_ELEM)
    return fail(FP4_ERR_ARG, "bad sweep kind %d", kind);
  if (n != kLen[kind])
    return fail(FP4_ERR_ARG, "sweep kind %d needs %d thresholds (got %d)", kind, kLen[kind], n);
  if (!thresholds || !result) return fail(FP4_ERR_ARG, "thresholds/result is null");
  if (reinterpret_cast<uintptr_t>(result) & 7u) return fail(FP4_ERR_ARG, "result must be 8-byte aligned");
  return device_status(fp4lib::launch_selftest_sweep(kind, thresholds, n, result,
                                                     static_cast<hipStream_t>(stream)),
                       "fp4_selftest_sweep launch");
}

FP4_EXPORT fp4_status fp4_selftest_gemm_decode(fp4_format format, uint16_t* out, void* stream) {
  if (format != FP4_NVFP4 && format != FP4_UE5M3)
    return fail(FP4_ERR_ARG, "gemm decode needs NVFP4 or UE5M3 (format %d)", (int)format);
  if (!out || (reinterpret_cast<uintptr_t>(out) & 1u)) return fail(FP4_ERR_ARG, "out is null or misaligned");
  return device_status(fp4lib::launch_selftest_gemm_decode(format, out,
                                                           static_cast<hipStream_t>(stream)),
                       "fp4_selftest_gemm_decode launch");
}
