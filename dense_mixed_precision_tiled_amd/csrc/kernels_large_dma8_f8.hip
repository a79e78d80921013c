// Kernel instantiations for the "fp8_large_dma8" tile-table entry (eight-wave
// LDS-DMA K loop, 32x32x64 MFMA, OCP fp8 E4M3 inputs; every operand
// layout), in a translation unit of its own so the library builds in
// parallel.
#include "gemm_configs.hpp"

namespace libgemm {
hipError_t launch_large_dma8_f8(const Params &p, int akc, int bkc, dim3 grid, hipStream_t s) {
    return launch_dma_layouts<CfgLargeDma8F8, IT_FP8>(p, akc, bkc, grid, s);
}
}  // namespace libgemm
