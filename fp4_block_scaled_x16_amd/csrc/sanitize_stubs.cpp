// Host-only stand-ins for the kernel launchers, linked with fp4_api.cpp into
// the AddressSanitizer / UndefinedBehaviorSanitizer build of the C ABI's
// validation code (build.py build_sanitized).  That build runs the
// argument-checking tests, which never reach a device: any call that passes
// validation reports "no device" here instead of launching.
#include <hip/hip_runtime.h>

#include "fp4_internal.hpp"

namespace fp4lib {

int device_cu_count() { return 256; }
int64_t grid_cap(int per_cu) { return 256 * static_cast<int64_t>(per_cu); }
int gemm_tile_rows_forced() { return 0; }
void set_launch_geometry(int, int) {}

hipError_t launch_amax(const uint16_t*, int64_t, int64_t, int64_t, int, int, const uint32_t (&)[4],
                       float*, hipStream_t, float*, bool) {
  return hipErrorNoDevice;
}
hipError_t launch_quant_row(const QuantArgs&, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_quant_row_scoped(const QuantArgs&, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_quant_col(const QuantArgs&, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_quant_2d(const QuantArgs&, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_quant_mx8(const QuantArgs&, bool, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_dequant_mx8(int, const uint8_t*, const uint8_t*, int64_t, int64_t, void*, int,
                              hipStream_t) {
  return hipErrorNoDevice;
}
hipError_t launch_quant_dual(const QuantArgs&, const QuantArgs&, hipStream_t) {
  return hipErrorNoDevice;
}
hipError_t launch_dequant(int, int, int, const uint8_t*, const uint8_t*, const float*, bool, int64_t,
                          int64_t, void*, int, hipStream_t) {
  return hipErrorNoDevice;
}
hipError_t launch_rht(const uint16_t*, int64_t, int64_t, int64_t, int, const uint32_t (&)[4], bool,
                      float*, hipStream_t) {
  return hipErrorNoDevice;
}
hipError_t launch_gemm(int, const GemmOperand&, const GemmOperand&, int64_t, int64_t, int64_t, void*,
                       int, int64_t, int, hipStream_t) {
  return hipErrorNoDevice;
}
hipError_t launch_selftest_sweep(int, const uint32_t*, int, uint64_t*, hipStream_t) {
  return hipErrorNoDevice;
}
hipError_t launch_selftest_gemm_decode(int, uint16_t*, hipStream_t) { return hipErrorNoDevice; }

}  // namespace fp4lib
