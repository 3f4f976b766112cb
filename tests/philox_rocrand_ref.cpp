// Reference Philox4x32-10 block outputs from rocRAND's public header, used to
// pin the CPU oracle's generator (tests/test_oracle_philox.py).  Reads lines
// "c0 c1 c2 c3 k0 k1" (decimal uint32) on stdin, prints the four output words.
#include <rocrand/rocrand_philox4x32_10.h>
#include <cstdio>

struct PhiloxBlock : rocrand_device::philox4x32_10_engine {
  using rocrand_device::philox4x32_10_engine::ten_rounds;   // protected in the engine
};

int main() {
  PhiloxBlock eng;
  unsigned c0, c1, c2, c3, k0, k1;
  while (std::scanf("%u %u %u %u %u %u", &c0, &c1, &c2, &c3, &k0, &k1) == 6) {
    uint4 r = eng.ten_rounds(uint4{c0, c1, c2, c3}, uint2{k0, k1});
    std::printf("%u %u %u %u\n", r.x, r.y, r.z, r.w);
  }
  return 0;
}
