// Device helpers shared by the quantizer translation units (quant.hip,
// quant_rowscope.hip): event counters, bf16 unpacking, block-scale
// selection, E2M1 encoding of one block, and the persistent-grid size.
#pragma once

#include <hip/hip_runtime.h>

#include <cmath>
#include <stdint.h>

#include "fp4_device.hpp"
#include "fp4_internal.hpp"

namespace fp4quant {

using namespace fp4dev;

// Same-address global atomics serialize (about 12 ns each on MI355X once
// more than a few hundred arrive), so every kernel runs a persistent grid
// of one or two workgroups per CU, reduces in LDS, and issues at most one
// atomic per workgroup and counter.

// ----------------------------------------------------------- counters --
// Reduce five per-thread event counts over the workgroup and add the
// nonzero totals to the caller's device counters (one atomic each).
template <int NT>
__device__ __forceinline__ void flush_counters(uint32_t (&c)[5], fp4_counters* out) {
  __shared__ uint32_t red[NT / 64][5];
#pragma unroll
  for (int k = 0; k < 5; ++k) {
    uint32_t v = c[k];
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    c[k] = v;
  }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) {
#pragma unroll
    for (int k = 0; k < 5; ++k) red[wave][k] = c[k];
  }
  __syncthreads();
  if (threadIdx.x < 5) {
    uint32_t t = 0;
#pragma unroll
    for (int w = 0; w < NT / 64; ++w) t += red[w][threadIdx.x];
    if (t) {
      unsigned long long* dst = reinterpret_cast<unsigned long long*>(out) + threadIdx.x;
      atomicAdd(dst, static_cast<unsigned long long>(t));
    }
  }
}

__device__ __forceinline__ void unpack8(const uint4& q, float* v) {
  const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = bf16_to_f32(w[i] & 0xFFFFu);
    v[2 * i + 1] = bf16_to_f32(w[i] >> 16);
  }
}

// Quantize BS values (already in fp32, in block order) with the encode
// scale; returns BS/8 packed code words (element i at bits 4 (i % 8) of
// word i / 8).  `idx0` is the output-layout index of element 0 (SR only).
// Counters, per lane: cnt[3] += #(|y| > 6); cnt[4] += NZX * #(x != 0) -
// #(code != 0), the number of nonzero inputs coded as zero (a zero input
// always codes to zero).  NZX = 2 lets one side of the dual quantizer count
// the nonzero inputs for both sides (NZX = 0 on the other).  Per-lane
// counts keep the tests on the vector unit; wave ballots would hold one
// 64-bit mask per test in scalar registers, which spill.
template <int BS, int RND, bool CNT, int NZX = 1>
__device__ __forceinline__ void encode_block(const float* v, float s_enc_l, uint64_t idx0,
                                             uint64_t seed, uint64_t offset, uint32_t* words,
                                             uint32_t (&cnt)[5]) {
  // SR on 32-element blocks: one Philox group at a time keeps registers low
  constexpr int kGroupUnroll = (RND == FP4_SR && BS > 16) ? 1 : BS / 8;
#pragma unroll kGroupUnroll
  for (int q = 0; q < BS / 8; ++q) {
    float y[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) y[i] = v[q * 8 + i] * s_enc_l;
    uint32_t word = 0;
    if constexpr (RND == FP4_SR) {
      word = e2m1_sr8(y, sr_words((idx0 >> 3) + q, seed, offset));
    } else {
      word = e2m1_rne_pair<0>(word, y[0], y[1]);
      word = e2m1_rne_pair<1>(word, y[2], y[3]);
      word = e2m1_rne_pair<2>(word, y[4], y[5]);
      word = e2m1_rne_pair<3>(word, y[6], y[7]);
    }
    words[q] = word;
    if constexpr (CNT) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        cnt[3] += fabsf(y[i]) > 6.0f ? 1u : 0u;
        if constexpr (NZX > 0) cnt[4] += v[q * 8 + i] != 0.0f ? static_cast<uint32_t>(NZX) : 0u;
      }
      cnt[4] -= nonzero_codes(word);
    }
  }
}

template <int FMT>
__device__ __forceinline__ uint32_t scale_for_block(float amax_b, float s_enc_g, float s_dec_g,
                                                    float& s_enc_l, uint32_t (&cnt)[5],
                                                    bool up, const float* enc_tab = nullptr) {
  if constexpr (FMT == kMX) {
    return block_scale_mx(amax_b, s_enc_l);
  } else {
    ScaleEvents ev{0, 0, 0};
    const uint32_t sc =
        block_scale_two_level<FMT>(amax_b, s_enc_g, s_dec_g, s_enc_l, ev, up, enc_tab);
    cnt[0] += ev.sat;
    cnt[1] += ev.under;
    cnt[2] += ev.sub;
    return sc;
  }
}

// The local encode scale of every block-scale code for one tensor scale,
// computed once per workgroup into LDS (thread c, c + NT, ...: code c);
// the caller synchronizes the workgroup before the first lookup.  Each
// block then reads its s_enc_L instead of dividing (the same value:
// enc_scale_of_code is block_scale_two_level's own arithmetic).
template <int FMT, int NT>
__device__ __forceinline__ void fill_enc_table(float* tab, float s_dec_g) {
  if constexpr (FMT != kMX) {
    for (int c = threadIdx.x; c < 256; c += NT) tab[c] = enc_scale_of_code<FMT>(c, s_dec_g);
  }
}

// Persistent grid: enough workgroups of `threads` for the work, at most
// per_cu per CU.
inline int grid_for(uint64_t work_items, int per_cu, int threads = 512) {
  const uint64_t want = (work_items + threads - 1) / threads;
  const uint64_t cap = static_cast<uint64_t>(fp4lib::grid_cap(per_cu));
  const uint64_t g = want < cap ? want : cap;
  return static_cast<int>(g ? g : 1);
}

// The RHT of size n (0 means 16) with the 128-bit sign mask s4.
inline RhtN make_rht(int n, const uint32_t (&s4)[4]) {
  RhtN r;
  r.n = n ? n : 16;
  r.scale = static_cast<float>(1.0 / std::sqrt(static_cast<double>(r.n)));
  for (int i = 0; i < 4; ++i) r.s[i] = s4[i];
  return r;
}

}  // namespace fp4quant
