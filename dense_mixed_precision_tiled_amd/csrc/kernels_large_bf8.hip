// Kernel instantiations for the "large_fp8" tile-table entry with OCP fp8 E5M2
// inputs (all operand layouts and load paths), in a translation unit of its
// own so the library builds in parallel.
#include "gemm_configs.hpp"

namespace libgemm {
hipError_t launch_large_bf8(const Params &p, int akc, int bkc, dim3 grid, hipStream_t s) {
    return launch_layouts<CfgLargeF8, IT_BF8>(p, akc, bkc, grid, s);
}
}  // namespace libgemm
