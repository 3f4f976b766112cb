// Block-scaled GEMM kernels (see launch_gemm).
#include <hip/hip_runtime.h>

#include "fp4_internal.hpp"

namespace fp4lib {

hipError_t launch_gemm(int, const GemmOperand&, const GemmOperand&, int64_t, int64_t, int64_t,
                       float*, int64_t, int, hipStream_t) {
  return hipErrorNotSupported;
}

}  // namespace fp4lib
