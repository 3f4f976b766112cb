// NVFP4 GEMM, codes by DMA: the 192-row output tiles (3 MFMA tiles of 32
// rows per wave).
#include "gemm_nv_dma.hpp"

namespace fp4gemm {

hipError_t launch_two_level_dma_192(int scv, const Params& p, hipStream_t s) {
  return launch_two_level_dma_mi<3>(scv, p, s);
}

}  // namespace fp4gemm
