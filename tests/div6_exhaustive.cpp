// Host check of fp4exact::div6_normal (the quantizers' amax_B / 6, NVFP4
// paper App. B.2 Eq. 2) against fp32 division on every fp32 pattern from
// 0 up to FLT_MAX.  Prints: mismatches inside [kDiv6Lo, kDiv6Hi], their
// smallest pattern, patterns checked there, and mismatches below kDiv6Lo
// (where the quantizers divide instead).
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "exact_div.hpp"

static float as_float(uint32_t b) { float x; memcpy(&x, &b, 4); return x; }
static uint32_t as_bits(float x) { uint32_t b; memcpy(&b, &x, 4); return b; }

int main() {
  const uint32_t lo = as_bits(fp4exact::kDiv6Lo), hi = as_bits(fp4exact::kDiv6Hi);
  unsigned long long bad = 0, checked = 0, below = 0;
  uint32_t first = 0xFFFFFFFFu;
#pragma omp parallel for schedule(static, 1 << 20) reduction(+ : bad, checked, below) reduction(min : first)
  for (int64_t i = 0; i <= (int64_t)hi; ++i) {
    const uint32_t b = (uint32_t)i;
    const float x = as_float(b);
    const bool same = as_bits(fp4exact::div6_normal(x)) == as_bits(x / 6.0f);
    if (b >= lo) {
      ++checked;
      if (!same) {
        ++bad;
        if (b < first) first = b;
      }
    } else if (!same) {
      ++below;
    }
  }
  printf("%llu %u %llu %llu\n", bad, first, checked, below);
  return 0;
}
