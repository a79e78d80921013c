// Kernel instantiations for the "skinny" tile-table entry (all input dtypes and
// operand layouts), in a translation unit of their own to build in parallel.
#include "gemm_configs.hpp"

namespace libgemm {
hipError_t launch_skinny(const Params &p, int bf, int akc, int bkc, dim3 grid, hipStream_t s) {
    return launch_cfg<CfgSkinny>(p, bf, akc, bkc, grid, s);
}
}  // namespace libgemm
