// Kernel instantiations for the "large8_i8" tile-table entry (int8 inputs, int32
// accumulator and output; all operand layouts and load paths), in a
// translation unit of its own so the library builds in parallel.
#include "gemm_configs.hpp"

namespace libgemm {
hipError_t launch_large8_i8(const Params &p, int, int akc, int bkc, dim3 grid, hipStream_t s) {
    return launch_layouts<CfgLarge8I8, IT_I8>(p, akc, bkc, grid, s);
}
}  // namespace libgemm
