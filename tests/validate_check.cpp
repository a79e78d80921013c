// Host check of the C ABI's argument validation (csrc/gemm_validate.hpp),
// built with g++ under AddressSanitizer and UndefinedBehaviorSanitizer by
// tests/test_sanitizers_cpu.py: every status the header documents, plus the
// extreme values where the arithmetic could overflow (dimensions near 2^31,
// leading dimensions near the 2^40 limit, addresses near the top of the
// address space).  Prints one line per failure and exits nonzero.
#include <stdint.h>
#include <stdio.h>

#include "gemm_validate.hpp"

using namespace libgemm_host;

static int g_fail = 0, g_checked = 0;

#define EXPECT(call, want)                                                          \
    do {                                                                            \
        const int got_ = (call);                                                    \
        ++g_checked;                                                                \
        if (got_ != (want)) {                                                       \
            printf("FAIL line %d: got %d want %d\n", __LINE__, got_, (int)(want)); \
            ++g_fail;                                                               \
        }                                                                           \
    } while (0)

static const void *P(uint64_t a) { return reinterpret_cast<const void *>((uintptr_t)a); }

int main() {
    const int R = GEMM_ROW_MAJOR, C = GEMM_COL_MAJOR;
    const uint64_t A = 0x10000000, B = 0x20000000, D = 0x40000000, Cp = 0x30000000;
    auto v = [&](int64_t M, int64_t N, int64_t K, uint64_t a, int64_t lda, int la, uint64_t b,
                 int64_t ldb, int lb, uint64_t c, int64_t ldc, uint64_t d, int64_t ldd, int in,
                 int acc, int out, const gemm_epilogue_t *e = nullptr, int satf = 0) {
        return validate(M, N, K, P(a), lda, la, P(b), ldb, lb, P(c), ldc, P(d), ldd, in, acc, out,
                        e, satf);
    };
    // accepted
    EXPECT(v(8, 8, 8, A, 8, R, B, 8, R, 0, 8, D, 8, GEMM_F16, GEMM_F32, GEMM_F32), GEMM_OK);
    EXPECT(v(8, 8, 8, A, 8, C, B, 8, C, D, 8, D, 8, GEMM_BF16, GEMM_F32, GEMM_BF16), GEMM_OK);
    EXPECT(v(8, 8, 8, A, 8, R, B, 8, R, 0, 8, D, 8, GEMM_F16, GEMM_F16, GEMM_F16), GEMM_OK);
    EXPECT(v(0, 8, 8, 0, 8, R, 0, 8, R, 0, 8, 0, 8, GEMM_F16, GEMM_F32, GEMM_F32), GEMM_OK);
    EXPECT(v(8, 8, 0, 0, 1, R, 0, 8, R, 0, 8, D, 8, GEMM_F16, GEMM_F32, GEMM_F32), GEMM_OK);
    EXPECT(v(8, 8, 8, A, 8, R, B, 8, C, 0, 8, D, 8, GEMM_I8, GEMM_I32, GEMM_I32), GEMM_OK);
    EXPECT(v(8, 8, 8, A, 8, R, B, 8, C, 0, 8, D, 8, GEMM_FP8_E4M3, GEMM_F32, GEMM_F16), GEMM_OK);
    // the largest dimensions and leading dimensions the contract allows
    const int64_t big = 0x7fffffff, ldmax = (int64_t)1 << 40;
    EXPECT(v(big, 1, 1, A, 1, R, 0x7f0000000000ull, 1, R, 0, 1, 0x7ff000000000ull, 1, GEMM_F16,
             GEMM_F32, GEMM_F32), GEMM_OK);
    EXPECT(v(2, 2, 2, A, ldmax, R, 0x7fff00000000ull, 2, R, 0, 2, A + ((uint64_t)1 << 40), 2,
             GEMM_F16, GEMM_F32, GEMM_F32), GEMM_ERR_ALIASING);  // D between A's two rows
    EXPECT(v(2, 2, 2, A, ldmax, R, 0x7fff00000000ull, 2, R, 0, 2, 0x7ffff0000000ull, 2, GEMM_F16,
             GEMM_F32, GEMM_F32), GEMM_OK);             // D past A's 2^41-byte extent
    EXPECT(v(2, 2, 2, 0x7fffff000000ull, ldmax, R, B, 2, R, 0, 2, D, 2, GEMM_F16, GEMM_F32,
             GEMM_F32), GEMM_OK);                       // an extent near the top of 64 bits
    // errors
    EXPECT(v(-1, 8, 8, A, 8, R, B, 8, R, 0, 8, D, 8, GEMM_F16, GEMM_F32, GEMM_F32), GEMM_ERR_INVALID_DIM);
    EXPECT(v(big + 1, 8, 8, A, 8, R, B, 8, R, 0, 8, D, 8, GEMM_F16, GEMM_F32, GEMM_F32), GEMM_ERR_INVALID_DIM);
    EXPECT(v(INT64_MIN, 8, 8, A, 8, R, B, 8, R, 0, 8, D, 8, GEMM_F16, GEMM_F32, GEMM_F32), GEMM_ERR_INVALID_DIM);
    EXPECT(v(8, 8, 8, A, 7, R, B, 8, R, 0, 8, D, 8, GEMM_F16, GEMM_F32, GEMM_F32), GEMM_ERR_INVALID_LD);
    EXPECT(v(8, 8, 8, A, ldmax + 1, R, B, 8, R, 0, 8, D, 8, GEMM_F16, GEMM_F32, GEMM_F32), GEMM_ERR_INVALID_LD);
    EXPECT(v(8, 8, 8, A, INT64_MAX, R, B, 8, R, 0, 8, D, 8, GEMM_F16, GEMM_F32, GEMM_F32), GEMM_ERR_INVALID_LD);
    EXPECT(v(8, 8, 8, A, 8, R, B, 8, R, Cp, 7, D, 8, GEMM_F16, GEMM_F32, GEMM_F32), GEMM_ERR_INVALID_LD);
    EXPECT(v(8, 8, 8, 0, 8, R, B, 8, R, 0, 8, D, 8, GEMM_F16, GEMM_F32, GEMM_F32), GEMM_ERR_NULL_PTR);
    EXPECT(v(8, 8, 8, A, 8, R, B, 8, R, 0, 8, 0, 8, GEMM_F16, GEMM_F32, GEMM_F32), GEMM_ERR_NULL_PTR);
    EXPECT(v(8, 8, 8, A, 8, R, B, 8, R, 0, 8, D, 8, GEMM_F32, GEMM_F32, GEMM_F32), GEMM_ERR_UNSUPPORTED);
    EXPECT(v(8, 8, 8, A, 8, R, B, 8, R, 0, 8, D, 8, GEMM_BF16, GEMM_F16, GEMM_F16), GEMM_ERR_UNSUPPORTED);
    EXPECT(v(8, 8, 8, A, 8, R, B, 8, R, 0, 8, D, 8, GEMM_I8, GEMM_I32, GEMM_F32), GEMM_ERR_UNSUPPORTED);
    EXPECT(v(8, 8, (int64_t)1 << 17, A, 1 << 17, R, B, 1 << 17, C, 0, 8, D, 8, GEMM_I8, GEMM_I32,
             GEMM_I32, nullptr, 1), GEMM_ERR_UNSUPPORTED);  // int8 satf needs K < 2^17
    EXPECT(v(8, 8, 8, A, 8, 2, B, 8, R, 0, 8, D, 8, GEMM_F16, GEMM_F32, GEMM_F32), GEMM_ERR_INVALID_LAYOUT);
    EXPECT(v(8, 8, 8, A, 8, R, B, 8, -1, 0, 8, D, 8, GEMM_F16, GEMM_F32, GEMM_F32), GEMM_ERR_INVALID_LAYOUT);
    EXPECT(v(8, 8, 8, A, 8, R, B, 8, R, 0, 8, A + 64, 8, GEMM_F16, GEMM_F32, GEMM_F32), GEMM_ERR_ALIASING);
    EXPECT(v(8, 8, 8, A, 8, R, B, 8, R, D + 4, 8, D, 8, GEMM_F16, GEMM_F32, GEMM_F32), GEMM_ERR_ALIASING);
    EXPECT(v(8, 8, 8, A, 8, R, B, 8, R, D, 9, D, 8, GEMM_F16, GEMM_F32, GEMM_F32), GEMM_ERR_ALIASING);
    // extended epilogue
    gemm_epilogue_t e = {1.0f, 1.0f, nullptr, GEMM_ACT_GELU, R, C};
    EXPECT(v(8, 8, 8, A, 8, R, B, 8, R, 0, 8, D, 8, GEMM_F16, GEMM_F32, GEMM_F32, &e), GEMM_OK);
    e.activation = 7;
    EXPECT(v(8, 8, 8, A, 8, R, B, 8, R, 0, 8, D, 8, GEMM_F16, GEMM_F32, GEMM_F32, &e), GEMM_ERR_UNSUPPORTED);
    e.activation = GEMM_ACT_RELU;
    e.layoutC = 5;
    EXPECT(v(8, 8, 8, A, 8, R, B, 8, R, Cp, 8, D, 8, GEMM_F16, GEMM_F32, GEMM_F32, &e), GEMM_ERR_INVALID_LAYOUT);
    e.layoutC = R;
    e.bias = reinterpret_cast<const float *>(P(D + 16));
    EXPECT(v(8, 8, 8, A, 8, R, B, 8, R, 0, 8, D, 8, GEMM_F16, GEMM_F32, GEMM_F32, &e), GEMM_ERR_ALIASING);
    e.bias = nullptr;
    e.alpha = 2.0f;
    EXPECT(v(8, 8, 8, A, 8, R, B, 8, C, 0, 8, D, 8, GEMM_I8, GEMM_I32, GEMM_I32, &e), GEMM_ERR_UNSUPPORTED);
    printf("checked %d calls, %d failures\n", g_checked, g_fail);
    return g_fail ? 1 : 0;
}
