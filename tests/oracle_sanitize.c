/* Drives every function of oracle/gemm_oracle.c on small and edge-case
 * problems (K = 0, one row or column, padded leading dimensions, in place,
 * sampled, product form, int8, fp8, every output type and epilogue), built
 * with gcc under AddressSanitizer and UndefinedBehaviorSanitizer by
 * tests/test_sanitizers_cpu.py.  Buffers are sized exactly to what the
 * definitions address, so any read or write past them is reported.  Exits
 * nonzero if a call rejects valid arguments. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int oracle_gemm(int64_t, int64_t, int64_t, const void *, int64_t, int, const void *, int64_t, int,
                const void *, int64_t, void *, int64_t, int, int, int, int, int);
int oracle_gemm_sampled(int64_t, int64_t, int64_t, const void *, int64_t, int, const void *,
                        int64_t, int, const void *, int64_t, int64_t, const int64_t *,
                        const int64_t *, void *, int, int, int, int, int);
int oracle_gemm_ex(int64_t, int64_t, int64_t, const void *, int64_t, int, const void *, int64_t,
                   int, const void *, int64_t, int, void *, int64_t, int, int, int, int, int,
                   double, double, const float *, int, int);
int oracle_gemm_i8(int64_t, int64_t, int64_t, const int8_t *, int64_t, int, const int8_t *, int64_t,
                   int, const int32_t *, int64_t, int, int32_t *, int64_t, int, int, int);
int oracle_decode_array(int, const void *, int64_t, double *);
int oracle_finish_array(int64_t, int64_t, const double *, const void *, int64_t, int, void *,
                        int64_t, int, int, int, double, double, const float *, int, int);
int oracle_finish_i8_array(int64_t, int64_t, const double *, const int32_t *, int64_t, int,
                           int32_t *, int64_t, int, int);
double oracle_element_fp64(int64_t, const void *, int64_t, int, const void *, int64_t, int,
                           const void *, int64_t, int, int, int64_t, int64_t);

static int fails = 0;
#define CHECK(x) do { if ((x) != 0) { printf("FAIL %s:%d %s\n", __FILE__, __LINE__, #x); ++fails; } } while (0)

/* elements addressed by an outer x inner matrix at stride ld */
static int64_t span(int64_t outer, int64_t inner, int64_t ld) { return outer ? (outer - 1) * ld + inner : 0; }

static void *alloc_exact(int64_t n, size_t es, unsigned fill) {
    void *p = malloc((size_t)(n > 0 ? n : 1) * es);
    memset(p, (int)fill, (size_t)(n > 0 ? n : 1) * es);
    return p;
}

int main(void) {
    const int64_t shapes[][3] = {{1, 1, 1}, {3, 5, 7}, {7, 3, 0}, {1, 9, 4}, {9, 1, 4}, {16, 16, 33}};
    const int outs[] = {0, 1, 2};  /* F32, F16, BF16 */
    for (unsigned si = 0; si < sizeof shapes / sizeof shapes[0]; ++si) {
        const int64_t M = shapes[si][0], N = shapes[si][1], K = shapes[si][2];
        for (int la = 0; la < 2; ++la)
            for (int lb = 0; lb < 2; ++lb)
                for (int oi = 0; oi < 3; ++oi) {
                    const int out = outs[oi], es = out == 0 ? 4 : 2;
                    const int64_t lda = (la == 0 ? K : M) + 1, ldb = (lb == 0 ? N : K) + 2;
                    const int64_t ldc = N + 3, ldd = N + 1;
                    const int64_t na = span(la == 0 ? M : K, la == 0 ? K : M, lda);
                    const int64_t nb = span(lb == 0 ? K : N, lb == 0 ? N : K, ldb);
                    uint16_t *A = alloc_exact(na, 2, 0x11), *B = alloc_exact(nb, 2, 0x22);
                    void *C = alloc_exact(span(M, N, ldc), es, 0x00);
                    void *D = alloc_exact(span(M, N, ldd), es, 0x00);
                    CHECK(oracle_gemm(M, N, K, A, lda, la, B, ldb, lb, C, ldc, D, ldd, 1, 0, out, 1, 2));
                    CHECK(oracle_gemm(M, N, K, A, lda, la, B, ldb, lb, D, ldd, D, ldd, 2, 0, out, 0, 1));
                    int64_t rows[3] = {0, M - 1, M / 2}, cols[3] = {N - 1, 0, N / 2};
                    void *smp = alloc_exact(3, es, 0);
                    CHECK(oracle_gemm_sampled(M, N, K, A, lda, la, B, ldb, lb, C, ldc, 3, rows, cols,
                                              smp, 1, 0, out, 0, 2));
                    float *bias = alloc_exact(N, 4, 0);
                    for (int lc = 0; lc < 2; ++lc)
                        for (int ld_ = 0; ld_ < 2; ++ld_)
                            for (int act = 0; act < 3; ++act) {
                                const int64_t ldc2 = (lc == 0 ? N : M) + 1, ldd2 = (ld_ == 0 ? N : M) + 2;
                                void *C2 = alloc_exact(span(lc == 0 ? M : N, lc == 0 ? N : M, ldc2), es, 0);
                                void *D2 = alloc_exact(span(ld_ == 0 ? M : N, ld_ == 0 ? N : M, ldd2), es, 0);
                                CHECK(oracle_gemm_ex(M, N, K, A, lda, la, B, ldb, lb, C2, ldc2, lc, D2,
                                                     ldd2, ld_, 1, 0, out, 1, 0.5, -2.0, bias, act, 2));
                                double *S = alloc_exact(M * N, 8, 0);
                                CHECK(oracle_finish_array(M, N, S, C2, ldc2, lc, D2, ldd2, ld_, out, 1, 0.5,
                                                          -2.0, bias, act, 3));
                                free(S); free(C2); free(D2);
                            }
                    double *dec = alloc_exact(na, 8, 0);
                    CHECK(oracle_decode_array(1, A, na, dec));
                    CHECK(oracle_decode_array(2, A, na, dec));
                    (void)oracle_element_fp64(K, A, lda, la, B, ldb, lb, C, ldc, 1, out, M - 1, N - 1);
                    free(dec); free(bias); free(smp); free(A); free(B); free(C); free(D);
                }
        /* int8 and fp8 */
        for (int la = 0; la < 2; ++la) {
            const int64_t lda = (la == 0 ? K : M) + 3, ldb = K + 1, ldd = N + 2, ldc = N;
            const int64_t na = span(la == 0 ? M : K, la == 0 ? K : M, lda), nb = span(N, K, ldb);
            int8_t *A = alloc_exact(na, 1, 0x81), *B = alloc_exact(nb, 1, 0x7f);
            int32_t *C = alloc_exact(span(M, N, ldc), 4, 0x44), *D = alloc_exact(span(M, N, ldd), 4, 0);
            CHECK(oracle_gemm_i8(M, N, K, A, lda, la, B, ldb, 1, C, ldc, 0, D, ldd, 0, 1, 2));
            CHECK(oracle_gemm_i8(M, N, K, A, lda, la, B, ldb, 1, NULL, ldc, 0, D, ldd, 0, 0, 1));
            double *S = alloc_exact(M * N, 8, 0);
            CHECK(oracle_finish_i8_array(M, N, S, C, ldc, 0, D, ldd, 0, 1));
            float *Df = alloc_exact(span(M, N, ldd), 4, 0);
            CHECK(oracle_gemm(M, N, K, A, lda, la, B, ldb, 1, NULL, ldc, Df, ldd, 5, 0, 0, 1, 2));
            CHECK(oracle_gemm(M, N, K, A, lda, la, B, ldb, 1, NULL, ldc, Df, ldd, 6, 0, 0, 0, 1));
            double *dec = alloc_exact(na, 8, 0);
            CHECK(oracle_decode_array(3, A, na, dec));
            CHECK(oracle_decode_array(5, A, na, dec));
            CHECK(oracle_decode_array(6, A, na, dec));
            free(dec); free(S); free(Df); free(A); free(B); free(C); free(D);
        }
    }
    /* empty problems touch nothing */
    CHECK(oracle_gemm(0, 5, 5, NULL, 5, 0, NULL, 5, 0, NULL, 5, NULL, 5, 1, 0, 0, 0, 1));
    CHECK(oracle_gemm(5, 0, 5, NULL, 5, 0, NULL, 5, 0, NULL, 5, NULL, 5, 1, 0, 0, 0, 1));
    printf("oracle sanitizer run: %d failures\n", fails);
    return fails ? 1 : 0;
}
