// Measurement kernels (not part of libgemm's boundary): the ceilings the GEMM
// is judged against on the machine it runs on.
//
//  - MFMA stream: every wave issues back-to-back v_mfma_f32_32x32x16_f16 or
//    v_mfma_f32_16x16x32_f16 on operands held in registers, over several
//    independent accumulators (so no MFMA waits for the previous one), with
//    no memory traffic in the loop.  Its rate is the matrix cores' sustained
//    peak for the operand data given (the clock under load depends on it).
//  - Copy: a grid-stride 16-byte load/store copy, the practical HBM rate for
//    streaming reads plus writes.
// The GEMM's roofline and the summaries of the measurements cite these rates
// next to the published peaks.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../../include/gemm_measure.h"

namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kAcc = 4;  // independent accumulators per wave

// Each lane loads its two 16-byte operands from `operands` (at lane-dependent
// offsets of a 64 KiB table), then runs `iters` rounds of kAcc MFMAs.
template <int MF>
__global__ void __launch_bounds__(512) mfma_stream_kernel(const u32x4 *operands, float *out,
                                                          int iters) {
    const int lane = threadIdx.x & 63;
    const int wave = (blockIdx.x * (blockDim.x / 64) + threadIdx.x / 64) & 63;
    const u32x4 a = operands[(wave * 64 + lane) & 4095];
    const u32x4 b = operands[(wave * 64 + lane + 2048) & 4095];
    const f16x8 fa = __builtin_bit_cast(f16x8, a), fb = __builtin_bit_cast(f16x8, b);
    if constexpr (MF == 32) {
        f32x16 acc[kAcc] = {};
        for (int it = 0; it < iters; ++it) {
#pragma unroll
            for (int q = 0; q < kAcc; ++q)
                acc[q] = __builtin_amdgcn_mfma_f32_32x32x16_f16(fa, fb, acc[q], 0, 0, 0);
        }
        float s = 0.0f;
#pragma unroll
        for (int q = 0; q < kAcc; ++q)
#pragma unroll
            for (int e = 0; e < 16; ++e) s += acc[q][e];
        out[blockIdx.x * blockDim.x + threadIdx.x] = s;
    } else {
        f32x4 acc[2 * kAcc] = {};
        for (int it = 0; it < iters; ++it) {
#pragma unroll
            for (int q = 0; q < 2 * kAcc; ++q)
                acc[q] = __builtin_amdgcn_mfma_f32_16x16x32_f16(fa, fb, acc[q], 0, 0, 0);
        }
        float s = 0.0f;
#pragma unroll
        for (int q = 0; q < 2 * kAcc; ++q)
#pragma unroll
            for (int e = 0; e < 4; ++e) s += acc[q][e];
        out[blockIdx.x * blockDim.x + threadIdx.x] = s;
    }
}

__global__ void __launch_bounds__(256) copy_kernel(const u32x4 *src, u32x4 *dst, int64_t n) {
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
        dst[i] = src[i];
}

}  // namespace

extern "C" {

int gemm_measure_mfma_stream(int mfma, int blocks, int threads, int iters, const void *operands,
                             float *out, void *stream) {
    if ((mfma != 32 && mfma != 16) || blocks < 1 || iters < 1 || !operands || !out ||
        (threads != 256 && threads != 512))
        return -1;
    const dim3 grid((unsigned)blocks), block((unsigned)threads);
    hipStream_t s = static_cast<hipStream_t>(stream);
    const u32x4 *op = static_cast<const u32x4 *>(operands);
    void *args[] = {&op, &out, &iters};
    const void *k = mfma == 32 ? reinterpret_cast<const void *>(mfma_stream_kernel<32>)
                               : reinterpret_cast<const void *>(mfma_stream_kernel<16>);
    return hipLaunchKernel(k, grid, block, args, 0, s) == hipSuccess ? 0 : -2;
}

int64_t gemm_measure_mfma_flops(int mfma, int blocks, int threads, int iters) {
    // every MFMA of either shape is 2 * 16384 multiply-adds per 64-lane wave
    // (32x32x16 = 16x16x32 * 2 = 16384 MACs; the 16x16 loop issues twice as
    // many): kAcc * 32768 FLOP per wave and round
    (void)mfma;
    return (int64_t)blocks * (threads / 64) * iters * kAcc * 32768;
}

int gemm_measure_copy(const void *src, void *dst, int64_t bytes, void *stream) {
    if (!src || !dst || bytes < 0 || bytes % 16) return -1;
    const int64_t n = bytes / 16;
    int64_t blocks = (n + 255) / 256;
    if (blocks > 8192) blocks = 8192;
    if (blocks < 1) return 0;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const u32x4 *sp = static_cast<const u32x4 *>(src);
    u32x4 *dp = static_cast<u32x4 *>(dst);
    int64_t nn = n;
    void *args[] = {&sp, &dp, &nn};
    return hipLaunchKernel(reinterpret_cast<const void *>(copy_kernel), dim3((unsigned)blocks),
                           dim3(256), args, 0, s) == hipSuccess ? 0 : -2;
}

}  // extern "C"
