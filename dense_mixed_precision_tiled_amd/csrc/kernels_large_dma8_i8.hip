// Kernel instantiations for the "i8_large_dma8" tile-table entry (eight-wave
// LDS-DMA K loop, 32x32x32 MFMA, int8 inputs, int32 accumulator and output;
// every operand layout), in a translation unit of its own so the library
// builds in parallel.
#include "gemm_configs.hpp"

namespace libgemm {
hipError_t launch_large_dma8_i8(const Params &p, int, int akc, int bkc, dim3 grid, hipStream_t s) {
    return launch_dma_layouts<CfgLargeDma8I8, IT_I8>(p, akc, bkc, grid, s);
}
}  // namespace libgemm
