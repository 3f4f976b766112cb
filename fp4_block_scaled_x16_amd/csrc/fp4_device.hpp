// Device arithmetic shared by the gfx950 quantizer kernels.
//
// Every function is written for bit-exact, order-fixed fp32 evaluation: the
// library is compiled with -ffp-contract=off, fp32 denormals preserved and
// correctly rounded fp32 division, so each '*', '/' and '+' below is one
// IEEE operation in the order written.
//
// Method (NVFP4 pretraining paper, arXiv:2509.25149):
//   App. B.1 Eq. 1  s_enc_G = 6 T / amax_X, s_dec_G = 1 / s_enc_G
//   App. B.2 Eq. 2  s_dec_L = amax_B / 6;  Eq. 3: scale = RNE(s_dec_L s_enc_G)
//                   s_enc_L = 1 / (scale * s_dec_G)
//   App. B.3 Eq. 4  code = Q(x * s_enc_L)
//   App. B.4 / §3   MXFP4: power-of-two scale rounded up, no tensor scale
//   §4.4            stochastic rounding for gradients
//   App. C          16-point Hadamard rotation, H_r = D_r H
// Conventions the pages leave open (clamps, tie handling, sign of zero, the
// random-bit layout) are fixed in include/fp4.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "exact_div.hpp"

namespace fp4dev {

constexpr float kFltMax = 3.40282346638528859812e+38f;

enum Fmt : int { kNV = 0, kUE = 1, kMX = 2 };

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// ---------------------------------------------------------------- scales --
// 8-bit scale with a 3-bit mantissa and exponent bias BIAS (E4M3: 7, max
// 448 = code 0x7E; UE5M3: 15, max 122880 = code 0xFF), round to nearest
// even, saturating at the maximum.  t >= 0 and finite.
template <int BIAS>
__device__ __forceinline__ uint32_t scale_m3_encode(float t, float tmax, uint32_t maxcode) {
  if (t >= tmax) return maxcode;
  constexpr float kMinNormal = (BIAS == 7) ? 0x1p-6f : 0x1p-14f;
  constexpr float kInvSubStep = (BIAS == 7) ? 0x1p9f : 0x1p17f;   // 1 / subnormal spacing
  if (t < kMinNormal) {
    // subnormal range: a multiple of the spacing, rint = half to even
    return static_cast<uint32_t>(__builtin_rintf(t * kInvSubStep));
  }
  const uint32_t b = __float_as_uint(t);
  // keep 3 mantissa bits, nearest-even on the 20 dropped bits; a carry
  // moves into the exponent field as it should
  const uint32_t r = b + 0x7FFFFu + ((b >> 20) & 1u);
  return (r >> 20) - ((127u - BIAS) << 3);
}

typedef short s16x2 __attribute__((ext_vector_type(2)));

// Four E4M3 element codes in one word, byte k = sign of y_k | E4M3 code of
// |y_k| rounded to nearest even (the grid scale_m3_encode<7> encodes:
// subnormal step 2^-9, largest value 448), through gfx950's packed FP8
// convert at unit scale.  Defined for |y_k| <= 448 only, where it agrees
// with scale_m3_encode<7> on every fp32 magnitude; callers scale a block so
// that no element exceeds 448.  Each convert fills the low half of a fresh
// word and the two halves are merged by a byte permute.
__device__ __forceinline__ uint32_t e4m3_pack4(float y0, float y1, float y2, float y3) {
  const s16x2 z = {0, 0};
  const s16x2 lo = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(z, y0, y1, 1.0f, false);
  const s16x2 hi = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(z, y2, y3, 1.0f, false);
  return __builtin_amdgcn_perm(__builtin_bit_cast(uint32_t, hi), __builtin_bit_cast(uint32_t, lo),
                               0x05040100u);
}

template <int BIAS>
__device__ __forceinline__ float scale_m3_decode(uint32_t code) {
  constexpr float kSubStep = (BIAS == 7) ? 0x1p-9f : 0x1p-17f;
  if (code < 8u) return static_cast<float>(code) * kSubStep;        // exact
  return __uint_as_float((code + ((127u - BIAS) << 3)) << 20);
}

__device__ __forceinline__ float ue8m0_decode(uint32_t code) {
  return code ? __uint_as_float(code << 23) : __uint_as_float(0x00400000u);  // 2^-127
}

// Tensor-level scales (Eq. 1).  amax = 0 -> s_enc = 1; overflow -> FLT_MAX.
__device__ __forceinline__ void global_scales(float amax, float target, float& s_enc,
                                              float& s_dec) {
  const float six_t = 6.0f * target;
  float e = 1.0f;
  if (amax != 0.0f) {
    e = six_t / amax;
    if (!(e <= kFltMax)) e = kFltMax;
  }
  s_enc = e;
  s_dec = 1.0f / e;
}

struct ScaleEvents {
  uint32_t sat, under, sub;
};

// Local encode scale of a block-scale code (Eq. 3's reciprocal):
// 1 / (s_hat * s_dec_G), clamped to FLT_MAX; 0 for the zero code.
template <int FMT>
__device__ __forceinline__ float enc_scale_of_code(uint32_t code, float s_dec_g) {
  const float s_hat = FMT == kNV ? scale_m3_decode<7>(code) : scale_m3_decode<15>(code);
  const float p = s_hat * s_dec_g;
  const float inv = fminf(1.0f / p, kFltMax);
  return code ? inv : 0.0f;
}

// Two-level block scale (Eqs. 2-3) -> scale code; s_enc_l receives the
// local encode scale (0 for a zero code, reciprocal clamped to FLT_MAX),
// read from `enc_tab` (enc_scale_of_code of every code for this s_dec_G)
// when the caller holds one, else computed.
template <int FMT>
// up: round the scale up instead of to nearest (truncation-free scaling,
// 2D-block FP4 page): the nearest code, moved one code up when its value is
// below t (the codes of both formats are ascending in value).
__device__ __forceinline__ uint32_t block_scale_two_level(float amax_b, float s_enc_g,
                                                          float s_dec_g, float& s_enc_l,
                                                          ScaleEvents& ev, bool up = false,
                                                          const float* enc_tab = nullptr) {
  // amax_B / 6 rounded as fp32 division rounds it; the multiply-and-correct
  // form holds on [2^-125, FLT_MAX] (every input checked on the host), a
  // branch divides below it and for inf / NaN (blocks that small are rare)
  float s_dec_l;
  if (amax_b >= fp4exact::kDiv6Lo && amax_b <= fp4exact::kDiv6Hi) [[likely]]
    s_dec_l = fp4exact::div6_normal(amax_b);
  else
    s_dec_l = amax_b / 6.0f;
  float t = s_dec_l * s_enc_g;
  if (!(t <= kFltMax)) t = kFltMax;
  uint32_t code;
  if constexpr (FMT == kNV) {
    ev.sat += (t > 448.0f);
    code = scale_m3_encode<7>(t, 448.0f, 0x7Eu);
    if (up && code < 0x7Eu && scale_m3_decode<7>(code) < t) ++code;
  } else {
    ev.sat += (t > 122880.0f);
    code = scale_m3_encode<15>(t, 122880.0f, 0xFFu);
    if (up && code < 0xFFu && scale_m3_decode<15>(code) < t) ++code;
  }
  s_enc_l = enc_tab ? enc_tab[code] : enc_scale_of_code<FMT>(code, s_dec_g);
  ev.under += (amax_b > 0.0f) & (code == 0u);
  ev.sub += (code >= 1u) & (code <= 7u);
  return code;
}

// MXFP4 block scale (App. B.4): the smallest e with 6 * 2^e >= amax_B,
// clamped to [-127, 127]; a zero block takes -127.  Returns e + 127 and the
// exact encode scale 2^-e.
__device__ __forceinline__ uint32_t block_scale_mx(float amax_b, float& s_enc_l) {
  int e = -127;
  if (amax_b > 0.0f) {
    const uint32_t b = __float_as_uint(amax_b);
    const int E = static_cast<int>(b >> 23);
    const uint32_t man = b & 0x7FFFFFu;
    int k;        // floor(log2(amax))
    bool le;      // amax <= 1.5 * 2^k
    if (E == 0) {  // fp32 subnormal: amax = man * 2^-149
      const int lead_pos = 31 - __clz(man);
      k = lead_pos - 149;
      const uint32_t lead = 1u << lead_pos;
      le = man <= lead + (lead >> 1);
    } else {
      k = E - 127;
      le = man <= 0x400000u;
    }
    // 6 * 2^(k-2) = 1.5 * 2^k covers amax iff le; otherwise 6 * 2^(k-1) does
    e = le ? k - 2 : k - 1;
    e = e < -127 ? -127 : (e > 127 ? 127 : e);
  }
  const int ne = -e;   // encode exponent in [-127, 127]
  s_enc_l = ne >= -126 ? __uint_as_float(static_cast<uint32_t>(ne + 127) << 23)
                       : __uint_as_float(0x00400000u);
  return static_cast<uint32_t>(e + 127);
}

// ------------------------------------------------------------ elements --
// E2M1 round to nearest even of y (Eq. 4), |y| > 6 saturates to 6; the
// sign bit copies y's.  Returns the 4-bit code.
__device__ __forceinline__ uint32_t e2m1_rne(float y) {
  const uint32_t yb = __float_as_uint(y);
  const uint32_t sign = (yb >> 28) & 8u;
  const uint32_t b = yb & 0x7FFFFFFFu;
  const float m = __uint_as_float(b);
  // below 1 the grid is {0, 0.5, 1} with ties 0.25 -> 0 and 0.75 -> 1
  const uint32_t small = static_cast<uint32_t>(m > 0.25f) + static_cast<uint32_t>(m >= 0.75f);
  // in [1, 6) E2M1 is a float with one mantissa bit and fp32's binades:
  // round the fp32 mantissa to one bit, nearest-even, read exponent|bit
  const uint32_t r = b + 0x1FFFFFu + ((b >> 22) & 1u);
  const uint32_t big = (r >> 22) - 252u;
  uint32_t mag = m < 1.0f ? small : big;
  mag = m < 6.0f ? mag : 7u;
  return sign | mag;
}

// Two E2M1 codes by round to nearest even, saturating at 6, written into
// byte SEL of `word` (y0 in the low nibble).  gfx950's FP4 conversion with a
// unit scale computes exactly e2m1_rne: checked on all 2^32 - 2^24 + 2
// non-NaN fp32 inputs.
template <int SEL>
__device__ __forceinline__ uint32_t e2m1_rne_pair(uint32_t word, float y0, float y1) {
  return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(word, y0, y1, 1.0f, SEL);
}

// Number of nonzero magnitudes among the 8 codes of a packed word: adding 7
// to a nonzero 3-bit magnitude carries into the nibble's sign position.
__device__ __forceinline__ uint32_t nonzero_codes(uint32_t word) {
  return __builtin_popcount(((word & 0x77777777u) + 0x77777777u) & 0x88888888u);
}

// -------------------------------------------------------------- Philox --
// Philox4x32-10 (Salmon et al., SC'11): ten rounds of two 32x32->64
// multiplies, key advanced by the Weyl constants between rounds.
struct U4 {
  uint32_t x, y, z, w;
};

__device__ __forceinline__ U4 philox4x32_10(U4 c, uint32_t k0, uint32_t k1) {
  // The key is uniform: left visible, the compiler hoists all ten round keys
  // out of the kernels' loops and, short of scalar registers, parks them in
  // vector-register lanes, paying a v_readlane (and its hazard wait) per key
  // per round.  An empty asm makes the key opaque here, so the round keys are
  // recomputed with scalar adds, which issue beside the vector work.
  asm volatile("" : "+s"(k0), "+s"(k1));
#pragma unroll
  for (int i = 0; i < 10; ++i) {
    if (i) {
      k0 += 0x9E3779B9u;
      k1 += 0xBB67AE85u;
    }
    const uint64_t p0 = static_cast<uint64_t>(0xD2511F53u) * c.x;
    const uint64_t p1 = static_cast<uint64_t>(0xCD9E8D57u) * c.z;
    const uint32_t hi0 = static_cast<uint32_t>(p0 >> 32), lo0 = static_cast<uint32_t>(p0);
    const uint32_t hi1 = static_cast<uint32_t>(p1 >> 32), lo1 = static_cast<uint32_t>(p1);
    // three-way xors as one gfx950 bitop3 each (0x96: the parity table)
    c = U4{static_cast<uint32_t>(__builtin_amdgcn_bitop3_b32(hi1, c.y, k0, 0x96)), lo1,
           static_cast<uint32_t>(__builtin_amdgcn_bitop3_b32(hi0, c.w, k1, 0x96)), lo0};
  }
  return c;
}

// 16 random bits for 8 consecutive output indices 8g .. 8g+7.
__device__ __forceinline__ U4 sr_words(uint64_t g, uint64_t seed, uint64_t offset) {
  return philox4x32_10(U4{static_cast<uint32_t>(g), static_cast<uint32_t>(g >> 32),
                          static_cast<uint32_t>(offset), static_cast<uint32_t>(offset >> 32)},
                       static_cast<uint32_t>(seed), static_cast<uint32_t>(seed >> 32));
}


// Stochastic E2M1 rounding (§4.4) of y[0..7] into one code word (element i
// in nibble i).  Element i takes 16 random bits u from word i >> 1 of w: the
// upper half for even i, the lower half for odd i.  With lo the largest E2M1
// magnitude <= |y|, hi the next and f = (|y| - lo) / (hi - lo), the code
// rounds up iff u + floor(65536 f) >= 65536; |y| >= 6 gives 6 and the sign
// bit copies y's.
//
// gfx950's stochastic packed FP4 convert takes two values and a 32-bit
// random operand R; it adds bits 10..31 of R (first value) or bits 9..30
// (second value) to the first 22 bits of f and rounds up on a carry.  With
// u in the top 16 of those 22 bits and zeros below, the carry is exactly
// the rule above.  Each pair goes through the convert twice, once with the
// even element's bits placed for the first value (its code: the low nibble
// of byte 0) and once with the odd element's bits placed for the second
// value (the high nibble).  Only byte 0 of each result is used: the
// instruction keeps the destination's other bytes, which the builtin does
// not model.  A bitfield insert per pair and three byte permutes assemble
// the word.
typedef float f32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t e2m1_sr8(const float (&y)[8], const U4& w) {
  const uint32_t wd[4] = {w.x, w.y, w.z, w.w};
  uint32_t b[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const f32x2 p = {y[2 * k], y[2 * k + 1]};
    const uint32_t ev = __builtin_amdgcn_cvt_scalef32_sr_pk_fp4_f32(0u, p, wd[k] & 0xFFFF0000u, 1.0f, 0);
    const uint32_t od = __builtin_amdgcn_cvt_scalef32_sr_pk_fp4_f32(0u, p, wd[k] << 15, 1.0f, 0);
    b[k] = (ev & 0x0Fu) | (od & 0xF0u);
  }
  // v_perm_b32: bytes 0-3 select from the second operand, 4-7 from the
  // first, 0x0C gives a zero byte
  const uint32_t b01 = __builtin_amdgcn_perm(b[1], b[0], 0x0C0C0400u);
  const uint32_t b23 = __builtin_amdgcn_perm(b[3], b[2], 0x0C0C0400u);
  return __builtin_amdgcn_perm(b23, b01, 0x05040100u);
}

// ----------------------------------------------------------------- RHT --
// (1/4) D_r H16 v: Walsh-Hadamard butterflies with strides 1, 2, 4, 8
// (each (a, b) -> (a + b, a - b)), exact 1/4, then output i negated when bit
// i of `signs` is set (H_r = D_r H flips rows of H, App. C).
__device__ __forceinline__ void rht16(float (&v)[16], uint32_t signs) {
#pragma unroll
  for (int h = 1; h < 16; h <<= 1) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if ((i & h) == 0) {
        const float a = v[i], b = v[i + h];
        v[i] = a + b;
        v[i + h] = a - b;
      }
    }
  }
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const float q = v[i] * 0.25f;
    v[i] = ((signs >> i) & 1u) ? -q : q;
  }
}

// Byte offset of the scale of (row r, block j) in the TILED scale layout:
// 2 KiB atoms of 8 consecutive blocks x 256 consecutive rows, row by row,
// kg = ceil(blocks per row / 8) atoms per 256-row band.
__host__ __device__ __forceinline__ uint64_t tiled_scale_offset(uint64_t r, uint64_t j,
                                                                uint64_t kg) {
  return (((r >> 8) * kg + (j >> 3)) << 11) + ((r & 255u) << 3) + (j & 7u);
}


// N-point variant (N in {4, 16, 32, 64, 128}): fl32(1/sqrt(N)) D_r H_N on
// groups of N consecutive rows of a column.  A lane holds 16 consecutive
// rows (one 1x16 block); for N > 16 the N / 16 lanes whose index bits 0-2
// (`grp`) differ only below N / 16 hold the rest of the group, and the
// butterflies with strides 16, 32, 64 run between them by xor shuffles
// (the lane with the bit clear holds the lower entry: a + b; its partner
// a - b).  Stride order 1, 2, 4, ... as in rht16; N = 4 runs strides 1, 2
// only (four independent 4-point transforms).  Every lane of an N-row
// group must be active.
struct RhtN {
  int n;
  float scale;          // fl32(1 / sqrt(n))
  uint32_t s[4];        // D_r: bit i of the 128-bit mask negates output row i
};

__device__ __forceinline__ void rht_n(float (&v)[16], const RhtN& r, int grp) {
#pragma unroll
  for (int h = 1; h < 16; h <<= 1) {
    if (h >= 4 && r.n < 16) break;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if ((i & h) == 0) {
        const float a = v[i], b = v[i + h];
        v[i] = a + b;
        v[i + h] = a - b;
      }
    }
  }
  for (int m = 1; 16 * m < r.n; m <<= 1) {
    const bool upper = (grp & m) != 0;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float o = __shfl_xor(v[i], m, 64);
      v[i] = upper ? o - v[i] : v[i] + o;
    }
  }
  // sign bits of this lane's rows: 16 consecutive bits from `base`
  const int base = r.n <= 16 ? 0 : ((grp & (r.n / 16 - 1)) << 4);
  const int wsel = base >> 5;
  const uint32_t word = wsel == 0 ? r.s[0] : wsel == 1 ? r.s[1] : wsel == 2 ? r.s[2] : r.s[3];
  const int lmask = r.n < 16 ? r.n - 1 : 15;
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    const float q = v[k] * r.scale;
    v[k] = ((word >> ((base & 31) + (k & lmask))) & 1u) ? -q : q;
  }
}
}  // namespace fp4dev
