// Kernel instantiations for the "tiny" tile-table entry with f16 inputs (all
// operand layouts and load paths), in a translation unit of their own so the
// library builds in parallel.
#include "gemm_configs.hpp"

namespace libgemm {
hipError_t launch_tiny_f16(const Params &p, int akc, int bkc, dim3 grid, hipStream_t s) {
    return launch_layouts<CfgTiny, IT_F16>(p, akc, bkc, grid, s);
}
}  // namespace libgemm
