/*
 * CPU oracle for the tiled mixed-precision matrix multiply-accumulate D = A x B + C.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the CPU
 * baseline leg of the benchmark load this library.  The GPU library never
 * includes, links or calls it, and this file includes nothing from the GPU
 * library: the two share no code.
 *
 * What it computes (the plain definition, nothing more):
 *   D[i,j] = round_out( sum_{k=0}^{K-1} A(i,k) * B(k,j)  +  C[i,j] ),  i < M, j < N
 * with the sum taken in fp64, k ascending, each product and each addition
 * rounded by plain IEEE double arithmetic (build with -ffp-contract=off so no
 * FMA is formed), then ONE rounding (round-to-nearest-even) to the output
 * dtype, then the saturate-to-finite rule if requested.
 *
 * Sources (the pages this follows):
 *  - Element definition C[i,j] = sum over k in [0,K) of A[i,k]*B[k,j]:
 *    "矩阵乘法优化可视化学习文档", section 1 "先建立心智模型"; the plain
 *    triple loop in section 3 "朴素实现为什么慢".
 *  - D = A*B + C with low-precision A, B and a high-precision C; D has the
 *    precision of C: "深入CUDA Tensor Core与WMMA…", section 2.2
 *    "核心运算：融合矩阵乘累加（MMA）".
 *  - Row-major offset i*N+j and column-major offset j*M+i, generalised to a
 *    leading dimension ld (stride between rows, resp. columns):
 *    same page, section 3.2 (the 2x3 example) and section 4.2 (ldm);
 *    "CUDA算子优化(5)：WMMA矩阵乘法", section "WMMA API解释" item (2).
 *  - In-place C = A*B + C and the satf rules (+Inf -> +MAX_NORM,
 *    -Inf -> -MAX_NORM, NaN -> +0): "CUDA算子优化(5)：WMMA矩阵乘法",
 *    section "WMMA API解释" item (5) mma_sync.
 *
 * Inputs may also be OCP fp8 (E4M3 or E5M2, one byte per element); see the
 * decoders below.
 *
 * Readings where the pages are silent or disagree (each also listed in the
 * design notes):
 *  - acc_dtype F16 ("HGEMM": fp16 accumulator, fp16 C and D) fixes the dtype of
 *    C, D and MAX_NORM; the value is still the exact-as-possible sum rounded
 *    once, like every other combination.
 *  - satf is applied once, to the final rounded output, with MAX_NORM the
 *    largest finite value of the output dtype.
 *  - C and D are row-major with ldc / ldd; C == NULL means C = 0.
 *  - Rounding is IEEE round-to-nearest-even; subnormals are kept.
 *
 * The extended form D = act(alpha * (A x B) + beta * C + bias), with C and D
 * row- or column-major, is at the end of the file with its own sources and
 * readings.
 *
 * Parity pins live in the CPU tests: exhaustive fp16 decode against numpy,
 * the RNE encoders against numpy float16/float32 casts and an exact rational
 * encoder, brute force of tiny GEMMs against exact rational sums, the 2x3
 * row/col-major example, integer closed forms, the in-place invariant and the
 * satf special cases.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { ORACLE_F32 = 0, ORACLE_F16 = 1, ORACLE_BF16 = 2, ORACLE_I8 = 3, ORACLE_I32 = 4,
       ORACLE_FP8_E4M3 = 5, ORACLE_FP8_E5M2 = 6 };
enum { ORACLE_ROW_MAJOR = 0, ORACLE_COL_MAJOR = 1 };

/* ---------------------------------------------------------------- decoding */

/* IEEE binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits. */
double oracle_decode_f16(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int m = h & 0x3ff;
    double v;
    if (e == 0)
        v = ldexp((double)m, -24); /* subnormal: m * 2^-24 */
    else if (e == 31)
        v = m ? NAN : INFINITY;
    else
        v = ldexp((double)(m + 1024), e - 25); /* (1024+m) * 2^(e-15-10) */
    return sign ? -v : v;
}

/* bfloat16: the upper 16 bits of an IEEE binary32. */
double oracle_decode_bf16(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/*
 * OCP 8-bit floating point (the formats the fp8 type lists of the pages refer
 * to, as defined by the OCP FP8 specification):
 *   E4M3: 1 sign, 4 exponent bits (bias 7), 3 fraction bits; no infinities,
 *         S.1111.111 is NaN, the largest finite value is 448;
 *   E5M2: 1 sign, 5 exponent bits (bias 15), 2 fraction bits; IEEE-style
 *         infinities (exponent 31, fraction 0) and NaNs.
 * Exponent field 0 holds subnormals.
 */
double oracle_decode_fp8_e4m3(uint8_t b)
{
    int sign = (b >> 7) & 1, e = (b >> 3) & 0xf, m = b & 7;
    double v;
    if (e == 0xf && m == 7)
        v = NAN;
    else if (e == 0)
        v = ldexp((double)m, -9);              /* m * 2^-3 * 2^(1-7) */
    else
        v = ldexp((double)(m + 8), e - 10);    /* (8+m) * 2^(e-7-3) */
    return sign ? -v : v;
}

double oracle_decode_fp8_e5m2(uint8_t b)
{
    int sign = (b >> 7) & 1, e = (b >> 2) & 0x1f, m = b & 3;
    double v;
    if (e == 0x1f)
        v = m ? NAN : INFINITY;
    else if (e == 0)
        v = ldexp((double)m, -16);             /* m * 2^-2 * 2^(1-15) */
    else
        v = ldexp((double)(m + 4), e - 17);    /* (4+m) * 2^(e-15-2) */
    return sign ? -v : v;
}

/* ---------------------------------------------------------------- encoding */

/* Round-half-to-even of a non-negative double to an integer-valued double. */
static double rne_integer(double n)
{
    double fl = floor(n);
    double frac = n - fl; /* exact: n and fl share the binade or fl == 0 */
    if (frac > 0.5)
        return fl + 1.0;
    if (frac < 0.5)
        return fl;
    return (fmod(fl, 2.0) == 0.0) ? fl : fl + 1.0;
}

/*
 * Encode x into a binary format with p fraction bits, exponent range
 * [emin, emax] for normal numbers, and bias = emax, rounding to nearest
 * even.  Values whose rounded magnitude exceeds the largest finite number
 * become infinities; tiny values become subnormals or signed zero.
 * Returns the bit pattern (sign | exponent | fraction).
 */
static uint32_t rne_encode(double x, int p, int emin, int emax)
{
    int ebits_shift = p;
    uint32_t sign = signbit(x) ? 1u : 0u;
    uint32_t sign_bit = sign << (p + (emax == 15 ? 5 : 8));
    uint32_t exp_all_ones = (emax == 15) ? 0x1fu : 0xffu;
    if (isnan(x))
        return sign_bit | (exp_all_ones << ebits_shift) | (1u << (p - 1));
    double a = fabs(x);
    if (isinf(a))
        return sign_bit | (exp_all_ones << ebits_shift);
    if (a == 0.0)
        return sign_bit;

    int e2;
    frexp(a, &e2);      /* a = f * 2^e2, f in [0.5, 1) */
    int e = e2 - 1;     /* 2^e <= a < 2^(e+1) */
    if (e < emin)
        e = emin;       /* subnormal range: fixed quantum 2^(emin-p) */
    double q = ldexp(1.0, e - p);     /* spacing of representable numbers */
    double n = rne_integer(a / q);    /* a/q is exact (power-of-two scale) */
    /* n is in [0, 2^(p+1)]; n == 2^(p+1) means carry into the next binade */
    if (n >= ldexp(1.0, p + 1)) {
        n = ldexp(1.0, p);
        e += 1;
    }
    if (n < ldexp(1.0, p)) {
        /* subnormal (only possible when e == emin) or zero */
        return sign_bit | (uint32_t)n;
    }
    if (e > emax)
        return sign_bit | (exp_all_ones << ebits_shift); /* overflow -> Inf */
    uint32_t biased = (uint32_t)(e + emax);
    uint32_t frac = (uint32_t)(n - ldexp(1.0, p));
    return sign_bit | (biased << ebits_shift) | frac;
}

uint16_t oracle_round_f16(double x) { return (uint16_t)rne_encode(x, 10, -14, 15); }

uint16_t oracle_round_bf16(double x) { return (uint16_t)rne_encode(x, 7, -126, 127); }

uint32_t oracle_round_f32_bits(double x) { return rne_encode(x, 23, -126, 127); }

/* -------------------------------------------------------- satf and MAX_NORM */

/* Largest finite value of each output dtype, as a bit pattern. */
static uint32_t max_norm_bits(int dtype)
{
    switch (dtype) {
    case ORACLE_F16: return 0x7bffu;       /* 65504 */
    case ORACLE_BF16: return 0x7f7fu;      /* (2 - 2^-7) * 2^127 */
    default: return 0x7f7fffffu;           /* FLT_MAX */
    }
}

/*
 * Round s (fp64) to the output dtype once, then apply satf to the rounded
 * value:  +Inf -> +MAX_NORM, -Inf -> -MAX_NORM, NaN -> +0.
 */
static uint32_t finish_element(double s, int out_dtype, int satf)
{
    uint32_t bits;
    int is_pos_inf, is_neg_inf, is_nan;
    if (out_dtype == ORACLE_F16) {
        bits = oracle_round_f16(s);
        is_nan = ((bits & 0x7c00u) == 0x7c00u) && (bits & 0x3ffu);
        is_pos_inf = bits == 0x7c00u;
        is_neg_inf = bits == 0xfc00u;
    } else if (out_dtype == ORACLE_BF16) {
        bits = oracle_round_bf16(s);
        is_nan = ((bits & 0x7f80u) == 0x7f80u) && (bits & 0x7fu);
        is_pos_inf = bits == 0x7f80u;
        is_neg_inf = bits == 0xff80u;
    } else {
        bits = oracle_round_f32_bits(s);
        is_nan = ((bits & 0x7f800000u) == 0x7f800000u) && (bits & 0x7fffffu);
        is_pos_inf = bits == 0x7f800000u;
        is_neg_inf = bits == 0xff800000u;
    }
    if (satf) {
        uint32_t mx = max_norm_bits(out_dtype);
        uint32_t sign = (out_dtype == ORACLE_F32) ? 0x80000000u : 0x8000u;
        if (is_pos_inf)
            bits = mx;
        else if (is_neg_inf)
            bits = sign | mx;
        else if (is_nan)
            bits = 0u;
    }
    return bits;
}

/* ------------------------------------------------------------ element access */

static double load_in(const void *base, int dtype, int64_t off)
{
    if (dtype == ORACLE_FP8_E4M3)
        return oracle_decode_fp8_e4m3(((const uint8_t *)base)[off]);
    if (dtype == ORACLE_FP8_E5M2)
        return oracle_decode_fp8_e5m2(((const uint8_t *)base)[off]);
    uint16_t h = ((const uint16_t *)base)[off];
    return dtype == ORACLE_BF16 ? oracle_decode_bf16(h) : oracle_decode_f16(h);
}

static double load_out(const void *base, int dtype, int64_t off)
{
    if (dtype == ORACLE_F32)
        return (double)((const float *)base)[off];
    uint16_t h = ((const uint16_t *)base)[off];
    return dtype == ORACLE_BF16 ? oracle_decode_bf16(h) : oracle_decode_f16(h);
}

static void store_out(void *base, int dtype, int64_t off, uint32_t bits)
{
    if (dtype == ORACLE_F32)
        ((uint32_t *)base)[off] = bits;
    else
        ((uint16_t *)base)[off] = (uint16_t)bits;
}

/* A(i,k): row-major -> A[i*lda + k]; col-major -> A[k*lda + i]. */
static int64_t a_offset(int layout, int64_t lda, int64_t i, int64_t k)
{
    return layout == ORACLE_ROW_MAJOR ? i * lda + k : k * lda + i;
}

/* B(k,j): row-major -> B[k*ldb + j]; col-major -> B[j*ldb + k]. */
static int64_t b_offset(int layout, int64_t ldb, int64_t k, int64_t j)
{
    return layout == ORACLE_ROW_MAJOR ? k * ldb + j : j * ldb + k;
}

typedef struct {
    int64_t M, N, K;
    const void *A; int64_t lda; int layoutA;
    const void *B; int64_t ldb; int layoutB;
    const void *C; int64_t ldc;
    void *D; int64_t ldd;
    int in_dtype, out_dtype, satf;
    /* sampled mode */
    int64_t nsamples;
    const int64_t *rows, *cols;
    void *out;
    /* work split */
    int64_t begin, end;
} job_t;

/* One output element, exactly the definition. */
static double dot_plus_c(const job_t *g, int64_t i, int64_t j)
{
    double s = 0.0;
    for (int64_t k = 0; k < g->K; ++k) {
        double a = load_in(g->A, g->in_dtype, a_offset(g->layoutA, g->lda, i, k));
        double b = load_in(g->B, g->in_dtype, b_offset(g->layoutB, g->ldb, k, j));
        double prod = a * b;
        s = s + prod;
    }
    if (g->C)
        s = s + load_out(g->C, g->out_dtype, i * g->ldc + j);
    return s;
}

/*
 * Full mode, rows [begin, end).  Row i's outputs are all computed (C is read)
 * before any of them is written, so C == D (in place) is safe.
 */
static void *full_worker(void *arg)
{
    const job_t *g = (const job_t *)arg;
    double *row = (double *)malloc(sizeof(double) * (size_t)(g->N > 0 ? g->N : 1));
    for (int64_t i = g->begin; i < g->end; ++i) {
        for (int64_t j = 0; j < g->N; ++j)
            row[j] = dot_plus_c(g, i, j);
        for (int64_t j = 0; j < g->N; ++j)
            store_out(g->D, g->out_dtype, i * g->ldd + j,
                      finish_element(row[j], g->out_dtype, g->satf));
    }
    free(row);
    return NULL;
}

static void *sample_worker(void *arg)
{
    const job_t *g = (const job_t *)arg;
    for (int64_t s = g->begin; s < g->end; ++s) {
        double v = dot_plus_c(g, g->rows[s], g->cols[s]);
        store_out(g->out, g->out_dtype, s, finish_element(v, g->out_dtype, g->satf));
    }
    return NULL;
}

static void run_split(job_t *proto, int64_t total, int nthreads, void *(*fn)(void *))
{
    if (nthreads < 1)
        nthreads = 1;
    if (nthreads > 256)
        nthreads = 256;
    if (total < nthreads)
        nthreads = total > 0 ? (int)total : 1;
    pthread_t th[256];
    job_t jobs[256];
    int started[256];
    for (int t = 0; t < nthreads; ++t) {
        jobs[t] = *proto;
        jobs[t].begin = total * t / nthreads;
        jobs[t].end = total * (t + 1) / nthreads;
        started[t] = (nthreads > 1) && pthread_create(&th[t], NULL, fn, &jobs[t]) == 0;
        if (!started[t])
            fn(&jobs[t]);
    }
    for (int t = 0; t < nthreads; ++t)
        if (started[t])
            pthread_join(th[t], NULL);
}

/*
 * Full oracle: writes D[i*ldd + j] for i < M, j < N and nothing else.
 * A, B: 16-bit patterns of in_dtype.  C, D: elements of out_dtype (fp32 or
 * 16-bit patterns).  acc_dtype only names the accumulator type of the call
 * (F32, or F16 for the HGEMM variant); the value computed is the same.
 * Returns 0, or -1 for an argument the definition does not cover.
 */
int oracle_gemm(int64_t M, int64_t N, int64_t K,
                const void *A, int64_t lda, int layoutA,
                const void *B, int64_t ldb, int layoutB,
                const void *C, int64_t ldc,
                void *D, int64_t ldd,
                int in_dtype, int acc_dtype, int out_dtype, int satf, int nthreads)
{
    (void)acc_dtype;
    if (M < 0 || N < 0 || K < 0)
        return -1;
    if (M == 0 || N == 0)
        return 0;
    job_t g;
    memset(&g, 0, sizeof g);
    g.M = M; g.N = N; g.K = K;
    g.A = A; g.lda = lda; g.layoutA = layoutA;
    g.B = B; g.ldb = ldb; g.layoutB = layoutB;
    g.C = C; g.ldc = ldc;
    g.D = D; g.ldd = ldd;
    g.in_dtype = in_dtype; g.out_dtype = out_dtype; g.satf = satf;
    run_split(&g, M, nthreads, full_worker);
    return 0;
}

/*
 * Sampled oracle: out[s] = D(rows[s], cols[s]) for s < nsamples, as out_dtype
 * elements packed densely.  Same arithmetic as oracle_gemm.
 */
int oracle_gemm_sampled(int64_t M, int64_t N, int64_t K,
                        const void *A, int64_t lda, int layoutA,
                        const void *B, int64_t ldb, int layoutB,
                        const void *C, int64_t ldc,
                        int64_t nsamples, const int64_t *rows, const int64_t *cols,
                        void *out,
                        int in_dtype, int acc_dtype, int out_dtype, int satf, int nthreads)
{
    (void)acc_dtype;
    if (M < 0 || N < 0 || K < 0 || nsamples < 0)
        return -1;
    for (int64_t s = 0; s < nsamples; ++s)
        if (rows[s] < 0 || rows[s] >= M || cols[s] < 0 || cols[s] >= N)
            return -1;
    job_t g;
    memset(&g, 0, sizeof g);
    g.M = M; g.N = N; g.K = K;
    g.A = A; g.lda = lda; g.layoutA = layoutA;
    g.B = B; g.ldb = ldb; g.layoutB = layoutB;
    g.C = C; g.ldc = ldc;
    g.in_dtype = in_dtype; g.out_dtype = out_dtype; g.satf = satf;
    g.nsamples = nsamples; g.rows = rows; g.cols = cols; g.out = out;
    run_split(&g, nsamples, nthreads, sample_worker);
    return 0;
}

/* Also exported for the pins: the fp64 pre-rounding value of one element. */
double oracle_element_fp64(int64_t K,
                           const void *A, int64_t lda, int layoutA,
                           const void *B, int64_t ldb, int layoutB,
                           const void *C, int64_t ldc,
                           int in_dtype, int out_dtype, int64_t i, int64_t j)
{
    job_t g;
    memset(&g, 0, sizeof g);
    g.K = K;
    g.A = A; g.lda = lda; g.layoutA = layoutA;
    g.B = B; g.ldb = ldb; g.layoutB = layoutB;
    g.C = C; g.ldc = ldc;
    g.in_dtype = in_dtype; g.out_dtype = out_dtype;
    return dot_plus_c(&g, i, j);
}

/* ===================================================== extended epilogue
 *
 * D = act( alpha * (A x B) + beta * C + bias ), then ONE rounding to the
 * output dtype, then satf; C and D each row- or column-major.
 *
 * Sources: the epilogue-fusion row of "矩阵乘法优化可视化学习文档" section 6
 * (bias, activation and scale applied before the write-back) and the Triton
 * notes of section 8 (bias/activation fused at the final store, with the
 * check that the fused result matches the unfused reference); the
 * accumulator load/store layouts mem_row_major / mem_col_major of
 * "CUDA算子优化(5)：WMMA矩阵乘法", section "WMMA API解释" items (3) and (4).
 *
 * Readings (the pages name bias, activation and scale but fix none of them):
 *  - scale is the usual pair alpha (on the product) and beta (on C);
 *    beta == 0 means C is not read at all;
 *  - bias is one fp32 value per output column j, added after the scaling;
 *  - activations: ReLU = max(x, 0) (NaN stays NaN, -0 becomes +0) and GELU in
 *    its erf form x * Phi(x) = x/2 * (1 + erf(x / sqrt 2)), with the limits
 *    GELU(+Inf) = +Inf and GELU(-Inf) = 0;
 *  - all of it in fp64 before the single final rounding.
 */
enum { ORACLE_ACT_NONE = 0, ORACLE_ACT_RELU = 1, ORACLE_ACT_GELU = 2 };

static double act_relu(double x)
{
    if (isnan(x))
        return x;
    return x > 0.0 ? x : 0.0;
}

static double act_gelu(double x)
{
    if (isnan(x))
        return x;
    if (isinf(x))
        return x > 0.0 ? x : 0.0;
    return 0.5 * x * (1.0 + erf(x / sqrt(2.0)));
}

static double apply_act(double x, int act)
{
    if (act == ORACLE_ACT_RELU)
        return act_relu(x);
    if (act == ORACLE_ACT_GELU)
        return act_gelu(x);
    return x;
}

/* C(i,j) / D(i,j): row-major -> [i*ld + j]; col-major -> [j*ld + i]. */
static int64_t cd_offset(int layout, int64_t ld, int64_t i, int64_t j)
{
    return layout == ORACLE_ROW_MAJOR ? i * ld + j : j * ld + i;
}

typedef struct {
    job_t base;
    int layoutC, layoutD;
    double alpha, beta;
    const float *bias;
    int act;
} job_ex_t;

/*
 * The epilogue of element (i,j) from its fp64 sum s, before the rounding:
 * act(alpha * s + beta * C(i,j) + bias[j]); C is read only when present and
 * beta != 0.
 */
static double epilogue_ex(double s, double alpha, double beta, const void *C, int out_dtype,
                          int64_t c_off, const float *bias, int64_t j, int act)
{
    double v = alpha * s;
    if (C && beta != 0.0)
        v = v + beta * load_out(C, out_dtype, c_off);
    if (bias)
        v = v + (double)bias[j];
    return apply_act(v, act);
}

/* One output element before the final rounding. */
static double element_ex(const job_ex_t *g, int64_t i, int64_t j)
{
    const job_t *b = &g->base;
    double s = 0.0;
    for (int64_t k = 0; k < b->K; ++k) {
        double a = load_in(b->A, b->in_dtype, a_offset(b->layoutA, b->lda, i, k));
        double bb = load_in(b->B, b->in_dtype, b_offset(b->layoutB, b->ldb, k, j));
        double prod = a * bb;
        s = s + prod;
    }
    return epilogue_ex(s, g->alpha, g->beta, b->C, b->out_dtype,
                       cd_offset(g->layoutC, b->ldc, i, j), g->bias, j, g->act);
}

/* Rows [begin, end): each row's values are computed before any is stored. */
static void *full_worker_ex(void *arg)
{
    const job_ex_t *g = (const job_ex_t *)arg;
    const job_t *b = &g->base;
    double *row = (double *)malloc(sizeof(double) * (size_t)(b->N > 0 ? b->N : 1));
    for (int64_t i = b->begin; i < b->end; ++i) {
        for (int64_t j = 0; j < b->N; ++j)
            row[j] = element_ex(g, i, j);
        for (int64_t j = 0; j < b->N; ++j)
            store_out(b->D, b->out_dtype, cd_offset(g->layoutD, b->ldd, i, j),
                      finish_element(row[j], b->out_dtype, b->satf));
    }
    free(row);
    return NULL;
}

static void *sample_worker_ex(void *arg)
{
    const job_ex_t *g = (const job_ex_t *)arg;
    const job_t *b = &g->base;
    for (int64_t s = b->begin; s < b->end; ++s) {
        double v = element_ex(g, b->rows[s], b->cols[s]);
        store_out(b->out, b->out_dtype, s, finish_element(v, b->out_dtype, b->satf));
    }
    return NULL;
}

static void run_split_ex(job_ex_t *proto, int64_t total, int nthreads, void *(*fn)(void *))
{
    if (nthreads < 1)
        nthreads = 1;
    if (nthreads > 256)
        nthreads = 256;
    if (total < nthreads)
        nthreads = total > 0 ? (int)total : 1;
    pthread_t th[256];
    job_ex_t jobs[256];
    int started[256];
    for (int t = 0; t < nthreads; ++t) {
        jobs[t] = *proto;
        jobs[t].base.begin = total * t / nthreads;
        jobs[t].base.end = total * (t + 1) / nthreads;
        started[t] = (nthreads > 1) && pthread_create(&th[t], NULL, fn, &jobs[t]) == 0;
        if (!started[t])
            fn(&jobs[t]);
    }
    for (int t = 0; t < nthreads; ++t)
        if (started[t])
            pthread_join(th[t], NULL);
}

static int fill_ex(job_ex_t *g, int64_t M, int64_t N, int64_t K,
                   const void *A, int64_t lda, int layoutA,
                   const void *B, int64_t ldb, int layoutB,
                   const void *C, int64_t ldc, int layoutC, int layoutD,
                   int in_dtype, int out_dtype, int satf,
                   double alpha, double beta, const float *bias, int act)
{
    if (M < 0 || N < 0 || K < 0)
        return -1;
    if (act < ORACLE_ACT_NONE || act > ORACLE_ACT_GELU)
        return -1;
    if ((layoutC != ORACLE_ROW_MAJOR && layoutC != ORACLE_COL_MAJOR) ||
        (layoutD != ORACLE_ROW_MAJOR && layoutD != ORACLE_COL_MAJOR))
        return -1;
    memset(g, 0, sizeof *g);
    job_t *b = &g->base;
    b->M = M; b->N = N; b->K = K;
    b->A = A; b->lda = lda; b->layoutA = layoutA;
    b->B = B; b->ldb = ldb; b->layoutB = layoutB;
    b->C = C; b->ldc = ldc;
    b->in_dtype = in_dtype; b->out_dtype = out_dtype; b->satf = satf;
    g->layoutC = layoutC; g->layoutD = layoutD;
    g->alpha = alpha; g->beta = beta; g->bias = bias; g->act = act;
    return 0;
}

/*
 * Full extended oracle: writes D(i,j) for i < M, j < N (at cd_offset) and
 * nothing else.  bias: N fp32 values or NULL.  Returns 0, or -1 for an
 * argument the definition does not cover.
 */
int oracle_gemm_ex(int64_t M, int64_t N, int64_t K,
                   const void *A, int64_t lda, int layoutA,
                   const void *B, int64_t ldb, int layoutB,
                   const void *C, int64_t ldc, int layoutC,
                   void *D, int64_t ldd, int layoutD,
                   int in_dtype, int acc_dtype, int out_dtype, int satf,
                   double alpha, double beta, const float *bias, int act, int nthreads)
{
    (void)acc_dtype;
    job_ex_t g;
    if (fill_ex(&g, M, N, K, A, lda, layoutA, B, ldb, layoutB, C, ldc, layoutC, layoutD,
                in_dtype, out_dtype, satf, alpha, beta, bias, act) != 0)
        return -1;
    if (M == 0 || N == 0)
        return 0;
    g.base.D = D;
    g.base.ldd = ldd;
    run_split_ex(&g, M, nthreads, full_worker_ex);
    return 0;
}

/* Sampled extended oracle: out[s] = D(rows[s], cols[s]), packed densely. */
int oracle_gemm_ex_sampled(int64_t M, int64_t N, int64_t K,
                           const void *A, int64_t lda, int layoutA,
                           const void *B, int64_t ldb, int layoutB,
                           const void *C, int64_t ldc, int layoutC,
                           int64_t nsamples, const int64_t *rows, const int64_t *cols,
                           void *out,
                           int in_dtype, int acc_dtype, int out_dtype, int satf,
                           double alpha, double beta, const float *bias, int act,
                           int nthreads)
{
    (void)acc_dtype;
    job_ex_t g;
    if (nsamples < 0 ||
        fill_ex(&g, M, N, K, A, lda, layoutA, B, ldb, layoutB, C, ldc, layoutC,
                ORACLE_ROW_MAJOR, in_dtype, out_dtype, satf, alpha, beta, bias, act) != 0)
        return -1;
    for (int64_t s = 0; s < nsamples; ++s)
        if (rows[s] < 0 || rows[s] >= M || cols[s] < 0 || cols[s] >= N)
            return -1;
    g.base.nsamples = nsamples;
    g.base.rows = rows;
    g.base.cols = cols;
    g.base.out = out;
    run_split_ex(&g, nsamples, nthreads, sample_worker_ex);
    return 0;
}

/* The fp64 value of one element after the activation, before the rounding. */
double oracle_element_ex_fp64(int64_t K,
                              const void *A, int64_t lda, int layoutA,
                              const void *B, int64_t ldb, int layoutB,
                              const void *C, int64_t ldc, int layoutC,
                              int in_dtype, int out_dtype,
                              double alpha, double beta, const float *bias, int act,
                              int64_t i, int64_t j)
{
    job_ex_t g;
    if (fill_ex(&g, 1, 1, K, A, lda, layoutA, B, ldb, layoutB, C, ldc, layoutC,
                ORACLE_ROW_MAJOR, in_dtype, out_dtype, 0, alpha, beta, bias, act) != 0)
        return NAN;
    return element_ex(&g, i, j);
}

/* The activation alone, for the pins. */
double oracle_activation(double x, int act) { return apply_act(x, act); }

/* ============================================================ int8 -> int32
 *
 * D(i,j) = to_int32( sum_k A(i,k) * B(k,j) + C(i,j) ), A and B int8 (two's
 * complement), C and D int32, each of C and D row- or column-major.
 *
 * Sources: the fragment type lists of "CUDA算子优化(5)：WMMA矩阵乘法" (A/B of
 * char / unsigned char with an int accumulator) and of "深入CUDA Tensor Core与
 * WMMA…" section 2.3 (INT8 on the matrix units); the sum itself is the element
 * definition of "矩阵乘法优化可视化学习文档" section 1.
 *
 * Readings: the sum is exact (int64 here: |a*b| <= 2^14, so any K < 2^49
 * fits); to_int32 wraps modulo 2^32 (two's complement), or with satf clamps
 * the exact value to [-2^31, 2^31 - 1] (the integer form of saturating to
 * the largest finite value); C == NULL means 0.
 */
static int32_t to_int32(int64_t v, int satf)
{
    if (satf) {
        if (v > INT32_MAX)
            return INT32_MAX;
        if (v < INT32_MIN)
            return INT32_MIN;
        return (int32_t)v;
    }
    return (int32_t)(uint32_t)(uint64_t)v; /* modulo 2^32 */
}

typedef struct {
    int64_t M, N, K;
    const int8_t *A; int64_t lda; int layoutA;
    const int8_t *B; int64_t ldb; int layoutB;
    const int32_t *C; int64_t ldc; int layoutC;
    int32_t *D; int64_t ldd; int layoutD;
    int satf;
    const int64_t *rows, *cols;
    int32_t *out;
    int64_t begin, end;
} job_i8_t;

static int64_t element_i8(const job_i8_t *g, int64_t i, int64_t j)
{
    int64_t s = 0;
    for (int64_t k = 0; k < g->K; ++k)
        s += (int64_t)g->A[a_offset(g->layoutA, g->lda, i, k)] *
             (int64_t)g->B[b_offset(g->layoutB, g->ldb, k, j)];
    if (g->C)
        s += g->C[cd_offset(g->layoutC, g->ldc, i, j)];
    return s;
}

static void *full_worker_i8(void *arg)
{
    const job_i8_t *g = (const job_i8_t *)arg;
    int64_t *row = (int64_t *)malloc(sizeof(int64_t) * (size_t)(g->N > 0 ? g->N : 1));
    for (int64_t i = g->begin; i < g->end; ++i) {
        for (int64_t j = 0; j < g->N; ++j)
            row[j] = element_i8(g, i, j);
        for (int64_t j = 0; j < g->N; ++j)
            g->D[cd_offset(g->layoutD, g->ldd, i, j)] = to_int32(row[j], g->satf);
    }
    free(row);
    return NULL;
}

static void *sample_worker_i8(void *arg)
{
    const job_i8_t *g = (const job_i8_t *)arg;
    for (int64_t s = g->begin; s < g->end; ++s)
        g->out[s] = to_int32(element_i8(g, g->rows[s], g->cols[s]), g->satf);
    return NULL;
}

static void run_split_i8(job_i8_t *proto, int64_t total, int nthreads, void *(*fn)(void *))
{
    if (nthreads < 1)
        nthreads = 1;
    if (nthreads > 256)
        nthreads = 256;
    if (total < nthreads)
        nthreads = total > 0 ? (int)total : 1;
    pthread_t th[256];
    job_i8_t jobs[256];
    int started[256];
    for (int t = 0; t < nthreads; ++t) {
        jobs[t] = *proto;
        jobs[t].begin = total * t / nthreads;
        jobs[t].end = total * (t + 1) / nthreads;
        started[t] = (nthreads > 1) && pthread_create(&th[t], NULL, fn, &jobs[t]) == 0;
        if (!started[t])
            fn(&jobs[t]);
    }
    for (int t = 0; t < nthreads; ++t)
        if (started[t])
            pthread_join(th[t], NULL);
}

/* Full int8 oracle: writes D(i,j) for i < M, j < N and nothing else. */
int oracle_gemm_i8(int64_t M, int64_t N, int64_t K,
                   const int8_t *A, int64_t lda, int layoutA,
                   const int8_t *B, int64_t ldb, int layoutB,
                   const int32_t *C, int64_t ldc, int layoutC,
                   int32_t *D, int64_t ldd, int layoutD, int satf, int nthreads)
{
    if (M < 0 || N < 0 || K < 0)
        return -1;
    if ((layoutC != ORACLE_ROW_MAJOR && layoutC != ORACLE_COL_MAJOR) ||
        (layoutD != ORACLE_ROW_MAJOR && layoutD != ORACLE_COL_MAJOR))
        return -1;
    if (M == 0 || N == 0)
        return 0;
    job_i8_t g;
    memset(&g, 0, sizeof g);
    g.M = M; g.N = N; g.K = K;
    g.A = A; g.lda = lda; g.layoutA = layoutA;
    g.B = B; g.ldb = ldb; g.layoutB = layoutB;
    g.C = C; g.ldc = ldc; g.layoutC = layoutC;
    g.D = D; g.ldd = ldd; g.layoutD = layoutD;
    g.satf = satf;
    run_split_i8(&g, M, nthreads, full_worker_i8);
    return 0;
}

/* Sampled int8 oracle: out[s] = D(rows[s], cols[s]). */
int oracle_gemm_i8_sampled(int64_t M, int64_t N, int64_t K,
                           const int8_t *A, int64_t lda, int layoutA,
                           const int8_t *B, int64_t ldb, int layoutB,
                           const int32_t *C, int64_t ldc, int layoutC,
                           int64_t nsamples, const int64_t *rows, const int64_t *cols,
                           int32_t *out, int satf, int nthreads)
{
    if (M < 0 || N < 0 || K < 0 || nsamples < 0)
        return -1;
    if (layoutC != ORACLE_ROW_MAJOR && layoutC != ORACLE_COL_MAJOR)
        return -1;
    for (int64_t s = 0; s < nsamples; ++s)
        if (rows[s] < 0 || rows[s] >= M || cols[s] < 0 || cols[s] >= N)
            return -1;
    job_i8_t g;
    memset(&g, 0, sizeof g);
    g.M = M; g.N = N; g.K = K;
    g.A = A; g.lda = lda; g.layoutA = layoutA;
    g.B = B; g.ldb = ldb; g.layoutB = layoutB;
    g.C = C; g.ldc = ldc; g.layoutC = layoutC;
    g.satf = satf;
    g.rows = rows; g.cols = cols; g.out = out;
    run_split_i8(&g, nsamples, nthreads, sample_worker_i8);
    return 0;
}

/* ============================================== product form (whole outputs)
 *
 * The same definitions for outputs too large for the per-element loops above:
 * the caller forms the fp64 sums S(i,j) = sum_k A(i,k) * B(k,j) with a
 * library fp64 matrix product of the exactly decoded operands (numpy's
 * matmul, in oracle/__init__.py), and the functions below do the rest.  The
 * library product sums in an order of its own, so S can differ from the
 * k-ascending sum of the loops above by fp64 rounding (at most about
 * K * 2^-53 * sum_k |A(i,k) * B(k,j)|); where every partial sum is exact in
 * fp64 (integer-valued and other short dyadic inputs) the two agree bit for
 * bit.  The epilogue, the single rounding and satf are the functions the
 * loops use.
 */

/* n elements of dtype (an input type, F32 or I32) decoded exactly to fp64. */
int oracle_decode_array(int dtype, const void *src, int64_t n, double *dst)
{
    if (n < 0)
        return -1;
    for (int64_t e = 0; e < n; ++e) {
        switch (dtype) {
        case ORACLE_F32: dst[e] = (double)((const float *)src)[e]; break;
        case ORACLE_F16: dst[e] = oracle_decode_f16(((const uint16_t *)src)[e]); break;
        case ORACLE_BF16: dst[e] = oracle_decode_bf16(((const uint16_t *)src)[e]); break;
        case ORACLE_I8: dst[e] = (double)((const int8_t *)src)[e]; break;
        case ORACLE_I32: dst[e] = (double)((const int32_t *)src)[e]; break;
        case ORACLE_FP8_E4M3: dst[e] = oracle_decode_fp8_e4m3(((const uint8_t *)src)[e]); break;
        case ORACLE_FP8_E5M2: dst[e] = oracle_decode_fp8_e5m2(((const uint8_t *)src)[e]); break;
        default: return -1;
        }
    }
    return 0;
}

typedef struct {
    int64_t M, N;
    const double *S;
    const void *C; int64_t ldc; int layoutC;
    void *D; int64_t ldd; int layoutD;
    int out_dtype, satf;
    double alpha, beta;
    const float *bias;
    int act;
    int64_t begin, end;
} job_fin_t;

/* Rows [begin, end): each row's values are formed before any is stored. */
static void *finish_worker(void *arg)
{
    const job_fin_t *g = (const job_fin_t *)arg;
    double *row = (double *)malloc(sizeof(double) * (size_t)(g->N > 0 ? g->N : 1));
    for (int64_t i = g->begin; i < g->end; ++i) {
        for (int64_t j = 0; j < g->N; ++j)
            row[j] = epilogue_ex(g->S[i * g->N + j], g->alpha, g->beta, g->C, g->out_dtype,
                                 cd_offset(g->layoutC, g->ldc, i, j), g->bias, j, g->act);
        for (int64_t j = 0; j < g->N; ++j)
            store_out(g->D, g->out_dtype, cd_offset(g->layoutD, g->ldd, i, j),
                      finish_element(row[j], g->out_dtype, g->satf));
    }
    free(row);
    return NULL;
}

/*
 * D(i,j) = satf(round(act(alpha * S(i,j) + beta * C(i,j) + bias[j]))) for
 * i < M, j < N; S is M x N, row-major and dense.  alpha = beta = 1, no bias
 * and no activation is the plain D = round(S + C) of oracle_gemm.  Nothing
 * else of D is written; C == D (same layout and ld) is the in-place update.
 */
int oracle_finish_array(int64_t M, int64_t N, const double *S,
                        const void *C, int64_t ldc, int layoutC,
                        void *D, int64_t ldd, int layoutD,
                        int out_dtype, int satf, double alpha, double beta,
                        const float *bias, int act, int nthreads)
{
    if (M < 0 || N < 0 || act < ORACLE_ACT_NONE || act > ORACLE_ACT_GELU)
        return -1;
    if ((layoutC != ORACLE_ROW_MAJOR && layoutC != ORACLE_COL_MAJOR) ||
        (layoutD != ORACLE_ROW_MAJOR && layoutD != ORACLE_COL_MAJOR))
        return -1;
    if (M == 0 || N == 0)
        return 0;
    job_fin_t g;
    memset(&g, 0, sizeof g);
    g.M = M; g.N = N; g.S = S;
    g.C = C; g.ldc = ldc; g.layoutC = layoutC;
    g.D = D; g.ldd = ldd; g.layoutD = layoutD;
    g.out_dtype = out_dtype; g.satf = satf;
    g.alpha = alpha; g.beta = beta; g.bias = bias; g.act = act;
    if (nthreads < 1)
        nthreads = 1;
    if (nthreads > 256)
        nthreads = 256;
    if (M < nthreads)
        nthreads = (int)M;
    pthread_t th[256];
    job_fin_t jobs[256];
    int started[256];
    for (int t = 0; t < nthreads; ++t) {
        jobs[t] = g;
        jobs[t].begin = M * t / nthreads;
        jobs[t].end = M * (t + 1) / nthreads;
        started[t] = (nthreads > 1) && pthread_create(&th[t], NULL, finish_worker, &jobs[t]) == 0;
        if (!started[t])
            finish_worker(&jobs[t]);
    }
    for (int t = 0; t < nthreads; ++t)
        if (started[t])
            pthread_join(th[t], NULL);
    return 0;
}

/*
 * int8 -> int32 from the sums: D(i,j) = to_int32(S(i,j) + C(i,j)).  S holds
 * the exact integer sums (the fp64 product of int8 values is exact while
 * K < 2^39: every partial sum stays below 2^53); values that are not
 * integers in that range are rejected (-1).
 */
int oracle_finish_i8_array(int64_t M, int64_t N, const double *S,
                           const int32_t *C, int64_t ldc, int layoutC,
                           int32_t *D, int64_t ldd, int layoutD, int satf)
{
    if (M < 0 || N < 0)
        return -1;
    if ((layoutC != ORACLE_ROW_MAJOR && layoutC != ORACLE_COL_MAJOR) ||
        (layoutD != ORACLE_ROW_MAJOR && layoutD != ORACLE_COL_MAJOR))
        return -1;
    const double lim = 9007199254740992.0; /* 2^53 */
    for (int64_t e = 0; e < M * N; ++e)
        if (!(S[e] > -lim && S[e] < lim) || S[e] != floor(S[e]))
            return -1;
    for (int64_t i = 0; i < M; ++i) {
        for (int64_t j = 0; j < N; ++j) {
            int64_t v = (int64_t)S[i * N + j];
            if (C)
                v += C[cd_offset(layoutC, ldc, i, j)];
            D[cd_offset(layoutD, ldd, i, j)] = to_int32(v, satf);
        }
    }
    return 0;
}
