/*
 * libgemm_measure — the measurement kernels the GEMM's roofline is read
 * against on the machine that runs it (not part of libgemm's boundary).
 *
 * The pages frame mixed-precision GEMM speed against the matrix units' peak
 * and the memory rate ("深入CUDA Tensor Core与WMMA…", section 1, the peak
 * comparison; "矩阵乘法优化可视化学习文档", section 10, the checklist: is the
 * kernel compute- or memory-bound).  These calls measure both ceilings
 * directly: published peaks assume a clock the chip does not hold under a
 * sustained MFMA load with random operands.
 *
 * gemm_measure_mfma_stream: `blocks` workgroups of `threads` (256: one wave
 *   per SIMD, 512: two) issue `iters` rounds of independent MFMAs (mfma = 32:
 *   v_mfma_f32_32x32x16_f16, 16: v_mfma_f32_16x16x32_f16) on fp16 operands
 *   read once from `operands` (device, 64 KiB: 4096 16-byte chunks, so the
 *   operand values -- random or constant -- are the caller's), writing one
 *   float per thread to `out` (device, blocks * threads floats).  Enqueued
 *   on `stream`; returns 0, -1 for a bad argument, -2 if the launch fails.
 * gemm_measure_mfma_flops: the FLOP count of such a launch.
 * gemm_measure_copy: dst[0, bytes) = src[0, bytes) with 16-byte loads and
 *   stores (bytes a multiple of 16; device buffers that do not overlap);
 *   returns 0, -1 or -2 as above.
 */
#ifndef GEMM_MEASURE_H
#define GEMM_MEASURE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

int gemm_measure_mfma_stream(int mfma, int blocks, int threads, int iters, const void *operands,
                             float *out, void *stream);
int64_t gemm_measure_mfma_flops(int mfma, int blocks, int threads, int iters);
int gemm_measure_copy(const void *src, void *dst, int64_t bytes, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* GEMM_MEASURE_H */
