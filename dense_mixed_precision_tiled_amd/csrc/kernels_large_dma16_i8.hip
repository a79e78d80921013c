// Kernel instantiations for the "i8_large_dma" tile-table entry (four-wave
// LDS-DMA K loop, 16x16x64 MFMA, int8 inputs, int32 accumulator and output;
// K-contiguous A and B only), in a translation unit of its own so the
// library builds in parallel.
#include "gemm_configs.hpp"

namespace libgemm {
hipError_t launch_large_dma16_i8(const Params &p, int, int akc, int bkc, dim3 grid,
                                 hipStream_t s) {
    // the host sends no other layout here
    if (!akc || !bkc) return hipErrorInvalidValue;
    return launch_dma_one<CfgLargeDmaI8_16, IT_I8, true, true>(p, grid, s);
}
}  // namespace libgemm
