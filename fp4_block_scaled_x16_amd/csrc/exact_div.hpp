// Correctly rounded fp32 quotient by the constant 6 (the block scale
// s_dec_L = amax_B / 6, NVFP4 paper App. B.2 Eq. 2) without the IEEE division
// sequence.  The fast form is plain C++ so that a host program can check it
// against fp32 division on every input it is used for.
#pragma once

#if defined(__HIPCC__)
#define FP4_HOST_DEVICE __host__ __device__
#else
#define FP4_HOST_DEVICE
#endif

namespace fp4exact {

// x * RN(1/6), corrected once by the fused remainder: q0 = x c,
// r = fma(-q0, 6, x) (exact), q = fma(r, c, q0).  Equal to RN(x / 6) for
// every x in [2^-125, FLT_MAX]; below 2^-125 the quotient is subnormal and
// the correction can round twice, so callers divide there (and for inf and
// NaN).
FP4_HOST_DEVICE inline float div6_normal(float x) {
  const float c = 0x1.555556p-3f;     // RN(1/6)
  const float q0 = x * c;
  return __builtin_fmaf(__builtin_fmaf(-q0, 6.0f, x), c, q0);
}

constexpr float kDiv6Lo = 0x1p-125f;                        // smallest input of div6_normal
constexpr float kDiv6Hi = 3.40282346638528859812e+38f;      // FLT_MAX

}  // namespace fp4exact
