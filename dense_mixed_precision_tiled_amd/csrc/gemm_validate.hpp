// Host-side argument validation of the C ABI (no HIP: the same code builds
// with a plain C++ compiler for the sanitizer test).  The checks follow the
// boundary's contract in include/libgemm.h: dimensions, leading dimensions,
// layouts, dtype combinations, null pointers and aliasing between D and the
// other operands.
#pragma once

#include <stdint.h>

#include "../../include/libgemm.h"

namespace libgemm_host {

inline bool is_fp8(int in_dtype) { return in_dtype == GEMM_FP8_E4M3 || in_dtype == GEMM_FP8_E5M2; }
inline int input_class(int in_dtype) { return in_dtype == GEMM_I8 ? 1 : (is_fp8(in_dtype) ? 2 : 0); }
inline int in_size(int in_dtype) { return (in_dtype == GEMM_I8 || is_fp8(in_dtype)) ? 1 : 2; }

inline int out_size(int dt) { return (dt == GEMM_F32 || dt == GEMM_I32) ? 4 : 2; }

// Byte range [lo, hi) of a matrix with `outer` lines of `inner` elements at
// stride ld; empty when either count is zero.
struct Range {
    unsigned __int128 lo, hi;
    bool empty() const { return hi <= lo; }
};

inline Range extent(const void *p, int64_t outer, int64_t inner, int64_t ld, int esize) {
    Range r;
    r.lo = (unsigned __int128)(uintptr_t)p;
    if (outer <= 0 || inner <= 0) {
        r.hi = r.lo;
        return r;
    }
    r.hi = r.lo + ((unsigned __int128)(outer - 1) * (unsigned __int128)ld +
                   (unsigned __int128)inner) * (unsigned __int128)esize;
    return r;
}

inline bool overlap(const Range &a, const Range &b) {
    return !a.empty() && !b.empty() && a.lo < b.hi && b.lo < a.hi;
}

inline const gemm_epilogue_t kPlainEpilogue = {1.0f, 1.0f, nullptr, GEMM_ACT_NONE, GEMM_ROW_MAJOR,
                                         GEMM_ROW_MAJOR};

inline int validate(int64_t M, int64_t N, int64_t K, const void *A, int64_t lda, int layoutA,
             const void *B, int64_t ldb, int layoutB, const void *C, int64_t ldc, const void *D,
             int64_t ldd, int in_dtype, int acc_dtype, int out_dtype,
             const gemm_epilogue_t *epi, int satf_arg) {
    if (!epi) epi = &kPlainEpilogue;
    const int64_t kMaxDim = 0x7fffffff;
    if (M < 0 || N < 0 || K < 0 || M > kMaxDim || N > kMaxDim || K > kMaxDim)
        return GEMM_ERR_INVALID_DIM;
    if (in_dtype == GEMM_I8 && acc_dtype == GEMM_I32 && out_dtype == GEMM_I32 && satf_arg &&
        K >= ((int64_t)1 << 17))
        return GEMM_ERR_UNSUPPORTED;
    auto layout_ok = [](int l) { return l == GEMM_ROW_MAJOR || l == GEMM_COL_MAJOR; };
    if (!layout_ok(layoutA) || !layout_ok(layoutB) || !layout_ok(epi->layoutC) ||
        !layout_ok(epi->layoutD))
        return GEMM_ERR_INVALID_LAYOUT;
    if (in_dtype != GEMM_F16 && in_dtype != GEMM_BF16 && in_dtype != GEMM_I8 && !is_fp8(in_dtype))
        return GEMM_ERR_UNSUPPORTED;
    if (in_dtype == GEMM_I8) {
        // int8 x int8 -> int32: the plain epilogue only (C/D layouts allowed);
        // satf clamps the exact sum, which the int32 accumulator holds only
        // for K < 2^17 (|a*b| <= 2^14)
        if (acc_dtype != GEMM_I32 || out_dtype != GEMM_I32) return GEMM_ERR_UNSUPPORTED;
        if (epi->alpha != 1.0f || (C && epi->beta != 1.0f && epi->beta != 0.0f) || epi->bias ||
            epi->activation != GEMM_ACT_NONE)
            return GEMM_ERR_UNSUPPORTED;
    } else if (acc_dtype == GEMM_F32) {
        if (out_dtype != GEMM_F32 && out_dtype != GEMM_F16 && out_dtype != GEMM_BF16)
            return GEMM_ERR_UNSUPPORTED;
    } else if (acc_dtype == GEMM_F16) {
        if (in_dtype != GEMM_F16 || out_dtype != GEMM_F16) return GEMM_ERR_UNSUPPORTED;
    } else {
        return GEMM_ERR_UNSUPPORTED;
    }
    if (epi->activation != GEMM_ACT_NONE && epi->activation != GEMM_ACT_RELU &&
        epi->activation != GEMM_ACT_GELU)
        return GEMM_ERR_UNSUPPORTED;
    const int64_t a_inner = layoutA == GEMM_ROW_MAJOR ? K : M;
    const int64_t a_outer = layoutA == GEMM_ROW_MAJOR ? M : K;
    const int64_t b_inner = layoutB == GEMM_ROW_MAJOR ? N : K;
    const int64_t b_outer = layoutB == GEMM_ROW_MAJOR ? K : N;
    const int64_t c_inner = epi->layoutC == GEMM_ROW_MAJOR ? N : M;
    const int64_t c_outer = epi->layoutC == GEMM_ROW_MAJOR ? M : N;
    const int64_t d_inner = epi->layoutD == GEMM_ROW_MAJOR ? N : M;
    const int64_t d_outer = epi->layoutD == GEMM_ROW_MAJOR ? M : N;
    // C is read only when present and beta != 0
    const bool reads_c = C && epi->beta != 0.0f;
    // leading dimensions: at least one line's worth, and small enough that
    // every element offset fits in 62 bits
    const int64_t kMaxLd = (int64_t)1 << 40;
    if (lda < 1 || lda < a_inner || lda > kMaxLd) return GEMM_ERR_INVALID_LD;
    if (ldb < 1 || ldb < b_inner || ldb > kMaxLd) return GEMM_ERR_INVALID_LD;
    if (ldd < 1 || ldd < d_inner || ldd > kMaxLd) return GEMM_ERR_INVALID_LD;
    if (reads_c && (ldc < 1 || ldc < c_inner || ldc > kMaxLd)) return GEMM_ERR_INVALID_LD;
    if (M == 0 || N == 0) return GEMM_OK;
    if (!D) return GEMM_ERR_NULL_PTR;
    if (K > 0 && (!A || !B)) return GEMM_ERR_NULL_PTR;

    const int osz = out_size(out_dtype);
    const Range rd = extent(D, d_outer, d_inner, ldd, osz);
    const int isz = in_size(in_dtype);
    const Range ra = K > 0 ? extent(A, a_outer, a_inner, lda, isz) : extent(A, 0, 0, 1, isz);
    const Range rb = K > 0 ? extent(B, b_outer, b_inner, ldb, isz) : extent(B, 0, 0, 1, isz);
    if (overlap(rd, ra) || overlap(rd, rb)) return GEMM_ERR_ALIASING;
    if (epi->bias && overlap(extent(epi->bias, 1, N, N, 4), rd)) return GEMM_ERR_ALIASING;
    if (reads_c) {
        const bool in_place = (C == D) && (ldc == ldd) && (epi->layoutC == epi->layoutD);
        if (!in_place && overlap(extent(C, c_outer, c_inner, ldc, osz), rd))
            return GEMM_ERR_ALIASING;
    }
    return GEMM_OK;
}

}  // namespace libgemm_host
