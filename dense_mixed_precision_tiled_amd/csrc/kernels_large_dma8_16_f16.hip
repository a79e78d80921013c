// Kernel instantiations for the "large_dma8_16" tile-table entry (LDS-DMA K loop,
// eight waves, 16x16x32 MFMA) with f16 inputs (all operand layouts), in a
// translation unit of their own so the library builds in parallel.
#include "gemm_configs.hpp"

namespace libgemm {
hipError_t launch_large_dma8_16_f16(const Params &p, int akc, int bkc, dim3 grid, hipStream_t s) {
    return launch_dma_layouts<CfgLargeDma8_16, IT_F16>(p, akc, bkc, grid, s);
}
}  // namespace libgemm
