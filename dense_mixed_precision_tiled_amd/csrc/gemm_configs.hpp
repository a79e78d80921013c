// The tile-shape table: one TileCfg per entry, and the launcher each kernel
// translation unit defines for it.
#pragma once

#include "gemm_kernels.hpp"

namespace libgemm {

// Large square-ish problems: 256x256 block tile, 2x2 waves of 128x128
// (4x4 MFMA 32x32x16 tiles per wave), BK 64, two LDS stages = 128 KiB.
using CfgLarge = TileCfg<256, 256, 64, 2, 2, 32>;
// Large problems, eight waves: the same 256x256x64 tile over 2x4 waves of
// 128x64 (4x2 MFMA tiles per wave), two waves per SIMD.  Each SIMD then
// alternates between two instruction streams, which hides LDS latency
// and issue gaps the single-wave schedule exposes.
using CfgLarge8 = TileCfg<256, 256, 64, 2, 4, 32>;
// Mid-size problems: 128x128, 2x2 waves of 64x64.
using CfgMedium = TileCfg<128, 128, 64, 2, 2, 32>;
// Small problems: 64x64, 2x2 waves of 32x32.
using CfgSmall = TileCfg<64, 64, 64, 2, 2, 32>;
// Tiny problems (fewer 64x64 tiles than half the CUs, e.g. 256^3): 32x32, one
// wave, so the grid has four times as many workgroups.
using CfgTiny = TileCfg<32, 32, 64, 1, 1, 32>;
// Skinny M <= 16: 16x128x128 tile, 1x4 waves of 16x32 with the 16x16x32
// MFMA, split-K so enough workgroups stream B.
using CfgSkinny = TileCfg<16, 128, 128, 1, 4, 16>;
// Large problems on the LDS-DMA K loop (gemm_dma_kernel): 256x256x64, 2x2
// waves of 128x128 (one per SIMD; 4x4 MFMA 32x32x16 tiles, accumulators in
// the AGPRs), operands loaded straight into LDS.  16-byte aligned operands
// only.
using CfgLargeDma = TileCfg<256, 256, 64, 2, 2, 32>;
// The same with the 16x16x32 MFMA (8x8 tiles of 16x16 per wave).
using CfgLargeDma16 = TileCfg<256, 256, 64, 2, 2, 16>;
// The LDS-DMA K loop with eight waves of 128x64 (two per SIMD; 128
// accumulators in AGPRs) and the 16x16x32 MFMA.  With two waves per SIMD
// the transposed LDS reads of an N- or M-contiguous operand keep up, so both
// operands arrive by DMA in every layout.  On par with the eight-wave
// register-staged tile at 4096^3 and slightly ahead with K-contiguous
// operands; an autotuning candidate.
using CfgLargeDma8_16 = TileCfg<256, 256, 64, 2, 4, 16>;

// int8 entries: the same tiles in bytes (BK = 128 int8 values per LDS row of
// 128 bytes), v_mfma_i32_32x32x32_i8 / v_mfma_i32_16x16x64_i8.
using CfgLarge8I8 = TileCfg<256, 256, 128, 2, 4, 32, 1>;
using CfgMediumI8 = TileCfg<128, 128, 128, 2, 2, 32, 1>;
using CfgSmallI8 = TileCfg<64, 64, 128, 2, 2, 32, 1>;
using CfgSkinnyI8 = TileCfg<16, 128, 256, 1, 4, 16, 1>;

// OCP fp8 entries (E4M3 or E5M2 A and B): the same tiles in bytes, two
// 16-byte chunks per lane and operand for v_mfma_scale_f32_32x32x64_f8f6f4 /
// 16x16x128 (scales 2^0), so two MFMA steps per 128-byte K-tile.  The large
// fp8 tile uses four waves (one per SIMD, 128x128 each): with two waves per
// SIMD the 32-byte fragments spill inside the K loop, and at 4096^3 the
// four-wave tile is ~25% faster.
using CfgLargeF8 = TileCfg<256, 256, 128, 2, 2, 32, 1, 2>;
using CfgMediumF8 = TileCfg<128, 128, 128, 2, 2, 32, 1, 2>;
using CfgSmallF8 = TileCfg<64, 64, 128, 2, 2, 32, 1, 2>;
using CfgSkinnyF8 = TileCfg<16, 128, 256, 1, 4, 16, 1, 2>;

// The LDS-DMA K loop for 8-bit operands (16-byte aligned rows, every layout):
// eight waves of 128x64 (two per SIMD, 128 accumulators each), 128 k values
// per K-tile; M- or N-contiguous operands are read with the transposing byte
// reads.  No operand passes through registers on its way to LDS, which
// leaves room for the fp8 MFMA's two-chunk fragments at two waves per SIMD.
using CfgLargeDma8I8 = TileCfg<256, 256, 128, 2, 4, 32, 1>;
using CfgLargeDma8F8 = TileCfg<256, 256, 128, 2, 4, 32, 1, 2>;
// Four waves of 128x128 (one per SIMD, 256 accumulators in AGPRs) with the
// int8 16x16x64 MFMA on the LDS-DMA K loop, both operands K-contiguous (the
// transposed byte reads serve the 32x32 MFMA only): 4096^3 ~10% faster than
// the eight-wave register-staged int8 tile.
using CfgLargeDmaI8_16 = TileCfg<256, 256, 128, 2, 2, 16, 1>;

typedef hipError_t (*launch_fn)(const Params &, int bf16, int a_kcontig, int b_kcontig,
                                dim3 grid, hipStream_t stream);

// one translation unit per (entry, input dtype): kernels_<entry>_<dtype>.hip
#define LIBGEMM_DECLARE_LAUNCH(name)                                                   \
    hipError_t launch_##name##_f16(const Params &, int, int, dim3, hipStream_t);     \
    hipError_t launch_##name##_bf16(const Params &, int, int, dim3, hipStream_t);    \
    inline hipError_t launch_##name(const Params &p, int bf, int akc, int bkc, dim3 grid, \
                                    hipStream_t s) {                                  \
        return bf ? launch_##name##_bf16(p, akc, bkc, grid, s)                        \
                  : launch_##name##_f16(p, akc, bkc, grid, s);                        \
    }
LIBGEMM_DECLARE_LAUNCH(large)
LIBGEMM_DECLARE_LAUNCH(large8)
LIBGEMM_DECLARE_LAUNCH(medium)
LIBGEMM_DECLARE_LAUNCH(small)
LIBGEMM_DECLARE_LAUNCH(skinny)
LIBGEMM_DECLARE_LAUNCH(large_dma)
LIBGEMM_DECLARE_LAUNCH(tiny)
LIBGEMM_DECLARE_LAUNCH(large_dma16)
LIBGEMM_DECLARE_LAUNCH(large_dma8_16)
#undef LIBGEMM_DECLARE_LAUNCH

// one translation unit per int8 entry: kernels_<entry>_i8.hip (the bf flag of
// launch_fn is ignored)
hipError_t launch_large8_i8(const Params &, int, int, int, dim3, hipStream_t);
hipError_t launch_medium_i8(const Params &, int, int, int, dim3, hipStream_t);
hipError_t launch_small_i8(const Params &, int, int, int, dim3, hipStream_t);
hipError_t launch_skinny_i8(const Params &, int, int, int, dim3, hipStream_t);
hipError_t launch_large_dma8_i8(const Params &, int, int, int, dim3, hipStream_t);
hipError_t launch_large_dma16_i8(const Params &, int, int, int, dim3, hipStream_t);

// fp8 entries, one translation unit per (entry, format): kernels_<entry>_f8.hip
// (E4M3) and kernels_<entry>_bf8.hip (E5M2); the bf flag of launch_fn selects
// E5M2
#define LIBGEMM_DECLARE_LAUNCH_F8(name)                                                  \
    hipError_t launch_##name##_f8(const Params &, int, int, dim3, hipStream_t);        \
    hipError_t launch_##name##_bf8(const Params &, int, int, dim3, hipStream_t);       \
    inline hipError_t launch_##name##_fp8(const Params &p, int e5m2, int akc, int bkc,  \
                                          dim3 grid, hipStream_t s) {                  \
        return e5m2 ? launch_##name##_bf8(p, akc, bkc, grid, s)                         \
                    : launch_##name##_f8(p, akc, bkc, grid, s);                         \
    }
LIBGEMM_DECLARE_LAUNCH_F8(large)
LIBGEMM_DECLARE_LAUNCH_F8(medium)
LIBGEMM_DECLARE_LAUNCH_F8(small)
LIBGEMM_DECLARE_LAUNCH_F8(skinny)
LIBGEMM_DECLARE_LAUNCH_F8(large_dma8)
#undef LIBGEMM_DECLARE_LAUNCH_F8

// Launch a kernel taking Params by value; the launch's own status is returned
// (not a sticky error left by an earlier call).
template <class Kern>
hipError_t launch_params(Kern kernel, dim3 grid, dim3 block, const Params &p, hipStream_t s) {
    Params arg = p;
    void *args[] = {&arg};
    return hipLaunchKernel(reinterpret_cast<const void *>(kernel), grid, block, args, 0, s);
}

template <class CF, int IT, bool AKC, bool BKC>
hipError_t launch_one(const Params &p, dim3 grid, hipStream_t s) {
    // the K loop masks k >= kend only when some slice ends inside a K-tile
    const bool ragged = (p.K % CF::BK) != 0 || (p.k_per_split % CF::BK) != 0;
    const dim3 block(CF::THREADS);
    if (!p.vec_ok)
        return launch_params(gemm_mfma_kernel<CF, IT, AKC, BKC, false, false>, grid, block, p, s);
    if (ragged)
        return launch_params(gemm_mfma_kernel<CF, IT, AKC, BKC, true, true>, grid, block, p, s);
    return launch_params(gemm_mfma_kernel<CF, IT, AKC, BKC, true, false>, grid, block, p, s);
}

// LDS-DMA kernels: vector operands only (the host never sends others here).
template <class CF, int IT, bool AKC, bool BKC>
hipError_t launch_dma_one(const Params &p, dim3 grid, hipStream_t s) {
    if (!p.vec_ok) return hipErrorInvalidValue;
    // Four-wave tiles with row-major A and B (B staged through registers)
    // run the RAGGED kernel for every K (its last-tile handling is a uniform
    // branch that whole K-tiles skip): its register allocation keeps the K
    // loop free of AGPR shuffles, while the other one moved ~100 values
    // through AGPRs per K-tile (4096^3: 163.5 -> 146-158 us).
    constexpr bool always = CF::WAVES_M * CF::WAVES_N == 4 && AKC && !BKC;
    const bool ragged = always || (p.K % CF::BK) != 0 || (p.k_per_split % CF::BK) != 0;
    const dim3 block(CF::THREADS);
    if (ragged) return launch_params(gemm_dma_kernel<CF, IT, AKC, BKC, true>, grid, block, p, s);
    if constexpr (!always)
        return launch_params(gemm_dma_kernel<CF, IT, AKC, BKC, false>, grid, block, p, s);
    return hipErrorInvalidValue;  // not reached
}

template <class CF, int IT>
hipError_t launch_dma_layouts(const Params &p, int akc, int bkc, dim3 grid, hipStream_t s) {
    if (akc)
        return bkc ? launch_dma_one<CF, IT, true, true>(p, grid, s)
                   : launch_dma_one<CF, IT, true, false>(p, grid, s);
    return bkc ? launch_dma_one<CF, IT, false, true>(p, grid, s)
               : launch_dma_one<CF, IT, false, false>(p, grid, s);
}

template <class CF, int IT>
hipError_t launch_layouts(const Params &p, int akc, int bkc, dim3 grid, hipStream_t s) {
    if (akc)
        return bkc ? launch_one<CF, IT, true, true>(p, grid, s)
                   : launch_one<CF, IT, true, false>(p, grid, s);
    return bkc ? launch_one<CF, IT, false, true>(p, grid, s)
               : launch_one<CF, IT, false, false>(p, grid, s);
}

}  // namespace libgemm
