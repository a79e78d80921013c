/*
 * libgemm — tiled mixed-precision matrix multiply-accumulate D = A x B + C
 * on AMD Instinct MI355X (gfx950), as hand-written HIP kernels behind a C ABI.
 *
 * The operation (sources, by page title and section):
 *  - D = A*B + C, fused multiply-accumulate with low-precision A, B and a
 *    high-precision accumulator; D has the precision of C:
 *    "深入CUDA Tensor Core与WMMA：从基础原理到高性能混合精度矩阵乘实战",
 *    section 2.2 "核心运算：融合矩阵乘累加（MMA）".
 *  - Element definition C[i,j] = sum over k in [0,K) of A[i,k]*B[k,j]:
 *    "矩阵乘法优化可视化学习文档", section 1 "先建立心智模型".
 *  - Row-major / column-major storage with a leading dimension (stride, in
 *    elements, between consecutive rows resp. columns): "深入CUDA Tensor Core
 *    与WMMA…", sections 3.2 (2x3 example) and 4.2 (ldm); "CUDA算子优化(5)：
 *    WMMA矩阵乘法", section "WMMA API解释" items (2) and (3).
 *  - In-place C = A*B + C, and satf (saturate to finite): +Inf -> +MAX_NORM,
 *    -Inf -> -MAX_NORM, NaN -> +0: "CUDA算子优化(5)：WMMA矩阵乘法",
 *    section "WMMA API解释" item (5) mma_sync.
 *  - fp16-accumulate HGEMM variant (fp16 A, B, C, D):
 *    "hgemm_mma_m16n8k16_naive_kernel", section 1.1 "m16n8k16 指令规格".
 *  - 8-bit float inputs (fp8): the per-architecture precision lists of
 *    "深入CUDA Tensor Core与WMMA…", section 2.3; here the OCP E4M3 and E5M2
 *    formats gfx950's matrix cores take.
 *  - int8 inputs with an int32 accumulator: the fragment type lists of
 *    "CUDA算子优化(5)：WMMA矩阵乘法" (char operands, int accumulator) and
 *    "深入CUDA Tensor Core与WMMA…", section 2.3 (INT8 on the matrix units).
 *
 * Readings where the pages leave a step open:
 *  - C and D are row-major (C(i,j) = C[i*ldc + j]); C has the output dtype.
 *  - acc_dtype GEMM_F16 selects the HGEMM variant: C, D and MAX_NORM are fp16.
 *    The sum itself is accumulated in fp32 (gfx950's f16 MFMAs accumulate in
 *    fp32) and rounded once to fp16, the accuracy the page on mixed precision
 *    asks for (section 7.1 "常见坑点", item 5).
 *  - satf is applied once, to the value rounded to out_dtype; MAX_NORM is the
 *    largest finite value of out_dtype.
 *  - Rounding to fp16 / bf16 is round-to-nearest-even.
 *  - Nothing outside rows [0,M) and columns [0,N) of D is written.  A and B
 *    are read in aligned 16-byte blocks (vector path) or element by element
 *    (other alignments): every block read holds at least one element of the
 *    M x K resp. K x N matrix, so bytes of the leading-dimension padding next
 *    to those elements (and up to 15 bytes past the last element) may be
 *    read, but never affect D; nothing else outside the matrices is read.
 *  - int8 (in_dtype GEMM_I8, acc and out GEMM_I32): the sum is exact; the
 *    result (+ C) wraps modulo 2^32, or with satf is clamped to the int32
 *    range.  satf needs K < 2^17, where the int32 accumulator cannot wrap.
 */
#ifndef LIBGEMM_H
#define LIBGEMM_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Storage order of A and B. */
typedef enum {
    GEMM_ROW_MAJOR = 0, /* X(r,c) = X[r*ld + c] */
    GEMM_COL_MAJOR = 1  /* X(r,c) = X[c*ld + r] */
} gemm_layout_t;

/* Element types. */
typedef enum {
    GEMM_F32 = 0,  /* IEEE binary32 */
    GEMM_F16 = 1,  /* IEEE binary16 */
    GEMM_BF16 = 2, /* bfloat16 (upper half of binary32) */
    GEMM_I8 = 3,   /* two's-complement 8-bit integer (A, B)  */
    GEMM_I32 = 4,  /* two's-complement 32-bit integer (C, D, accumulator) */
    GEMM_FP8_E4M3 = 5, /* OCP 8-bit float E4M3 (A, B): bias 7, max 448, NaN, no Inf */
    GEMM_FP8_E5M2 = 6  /* OCP 8-bit float E5M2 (A, B): bias 15, IEEE-style Inf/NaN */
} gemm_dtype_t;

/* Return codes.  GEMM_OK means "validated and enqueued". */
typedef enum {
    GEMM_OK = 0,
    GEMM_ERR_INVALID_DIM = -1,    /* M, N or K negative, or above 2^31-1        */
    GEMM_ERR_INVALID_LD = -2,     /* a leading dimension shorter than its matrix */
    GEMM_ERR_NULL_PTR = -3,       /* NULL A, B or D for a non-empty operation    */
    GEMM_ERR_UNSUPPORTED = -4,    /* dtype combination not provided              */
    GEMM_ERR_INVALID_LAYOUT = -5, /* layout not GEMM_ROW_MAJOR / GEMM_COL_MAJOR  */
    GEMM_ERR_ALIASING = -6,       /* D overlaps A or B, or C partially overlaps D */
    GEMM_ERR_HIP = -7,            /* the HIP runtime reported an error           */
    GEMM_ERR_INVALID_CONFIG = -8, /* gemm_run_config: no such config, or the
                                     config cannot run this problem            */
    GEMM_ERR_SCRATCH_TOO_SMALL = -9 /* gemm_run_noalloc: the split-K partial
                                     sums need more than its fixed scratch     */
} gemm_status_t;

/*
 * D = A x B + C on the device.
 *
 *   M, N, K      problem size: A is M x K, B is K x N, C and D are M x N.
 *                M == 0 or N == 0: nothing to do, returns GEMM_OK.
 *                K == 0: D = satf(round(C)) (or +0 when C is NULL).
 *   A, lda, layoutA   device pointer to in_dtype elements; lda >= K when
 *                row-major, >= M when col-major (and >= 1).
 *   B, ldb, layoutB   device pointer to in_dtype elements; ldb >= N when
 *                row-major, >= K when col-major (and >= 1).
 *   C, ldc       device pointer to out_dtype elements, row-major, ldc >= N;
 *                may be NULL (C = 0).  C == D with ldc == ldd is the in-place
 *                update C = A x B + C; any other overlap of C and D is rejected.
 *   D, ldd       device pointer to out_dtype elements, row-major, ldd >= N.
 *   in_dtype     GEMM_F16, GEMM_BF16, GEMM_FP8_E4M3, GEMM_FP8_E5M2 (A and B
 *                both of that type), or GEMM_I8 (A and B int8).
 *   acc_dtype    GEMM_F32 (out_dtype F32, F16 or BF16; any float input), or GEMM_F16 with
 *                in_dtype == out_dtype == GEMM_F16 (HGEMM), or GEMM_I32 with
 *                in_dtype GEMM_I8 and out_dtype GEMM_I32.
 *   out_dtype    dtype of C and D.
 *   satf         nonzero: +Inf -> +MAX_NORM, -Inf -> -MAX_NORM, NaN -> +0;
 *                for int32 output: clamp to [-2^31, 2^31-1] instead of wrapping
 *                (int8 with K >= 2^17 and satf: GEMM_ERR_UNSUPPORTED).
 *   stream       a hipStream_t (NULL = the null stream).  The work is enqueued
 *                on it; the call does not wait for it.
 *
 * Ownership: every pointer is owned by the caller and must stay valid until
 * the stream reaches the enqueued work.  Problems split along K (M <= 16),
 * and large calls (M*N*K >= 2^30) whose A or B misses the vector loads only
 * by alignment (that operand is first copied there with 16-byte lines), use
 * a device workspace the library owns: one per (device, stream) pair,
 * allocated with hipMalloc on first need and grown on demand.  A call holds
 * the workspace's lock from taking the buffer until all of its launches are
 * enqueued, so calls from several host threads on one stream are enqueued
 * one after the other; an outgrown buffer is never freed (work enqueued
 * earlier may still use it).  Workspaces are kept until the process exits.
 *
 * Errors: argument errors are detected on the host before anything is
 * enqueued, and nothing is written.  GEMM_ERR_HIP reports a launch or
 * allocation failure (the launch's own status, not an earlier error); D is
 * then not written, except that a call whose later launch fails has already
 * enqueued the earlier ones (an operand copy, a split-K slice kernel), which
 * write only the workspace.
 * Faults inside the kernels surface at the next synchronisation of the
 * stream.
 *
 * Speed: vector loads are used where A and B base pointers are 16-byte
 * aligned and lda, ldb are multiples of 16 bytes (the pages' ldm rule), in
 * every layout (operands contiguous along M or N are transposed on the way
 * to LDS); large calls with other operands copy them into the workspace
 * with 16-byte lines first (see Ownership), and the rest run correct
 * element-wise loads.  C and D
 * are read and written four elements at a time where their base pointers
 * are aligned to four elements, ldc and ldd are multiples of 4 and C is
 * row-major (and, for gemm_run_ex, a per-column bias is 16-byte aligned);
 * otherwise element by element.
 *
 * fp8 accuracy: gfx950's fp8 MFMA adds the products of each output in
 * groups of 8 consecutive k, aligned to the largest product of the group:
 * what lies below 2^-13 of that product is lost (measured, E4M3 and E5M2),
 * before the fp32 accumulation.  Each product is then off by less than
 * 2^-13 * max|a| * max|b|.  Products of inputs of similar magnitude, and
 * integer-valued inputs, come out exact.
 */
int gemm_run(int64_t M, int64_t N, int64_t K,
             const void *A, int64_t lda, int layoutA,
             const void *B, int64_t ldb, int layoutB,
             const void *C, int64_t ldc,
             void *D, int64_t ldd,
             int in_dtype, int acc_dtype, int out_dtype,
             int satf, void *stream);

/*
 * gemm_run without any device allocation, for callers that cannot allocate:
 * code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  Same arguments, validation and results as gemm_run (the same
 * kernels, bit-identical D), except for large calls whose operands gemm_run
 * would copy into its workspace for alignment: this call runs those with
 * element-wise loads instead (the same results to the stated tolerances;
 * slower).  Where gemm_run would take its split-K partial
 * sums from a workspace it allocates (M <= 16), this call uses a scratch
 * array of fixed size compiled into the library: 32 MiB of device memory per
 * GPU the library runs on, held until the process ends.  Problems whose
 * partial sums (splits * M * N * 4 bytes) exceed it return
 * GEMM_ERR_SCRATCH_TOO_SMALL before anything is enqueued (on a 256-CU
 * MI355X no problem needs more than about 17 MB).  Every call on a
 * GPU shares that GPU's scratch, and nothing guards it: calls that can
 * overlap on one GPU (other streams, other host threads) race on it and must
 * be ordered by the caller.  The scratch needs no clearing (each call writes
 * every partial sum it reads).  The call makes no hipMalloc, hipFree or other
 * allocating call; its first call on a device looks up the scratch's device
 * address (hipGetSymbolAddress), which allocates no memory of its own: the
 * scratch is part of the library's device code object.  The call enqueues
 * only kernel launches (no memset or copy nodes), so it can be captured into
 * a HIP graph once the device is initialised; a replay computes what the
 * captured call would (tested: replays between eager calls of both entry
 * points, bit-identical to the eager result).
 */
int gemm_run_noalloc(int64_t M, int64_t N, int64_t K,
                     const void *A, int64_t lda, int layoutA,
                     const void *B, int64_t ldb, int layoutB,
                     const void *C, int64_t ldc,
                     void *D, int64_t ldd,
                     int in_dtype, int acc_dtype, int out_dtype,
                     int satf, void *stream);

/* Static text for a gemm_status_t value ("unknown status" otherwise). */
const char *gemm_status_string(int status);

/*
 * The tile-shape table.  Each entry is one tiling (block tile, wave grid,
 * MFMA shape, split-K policy); the dispatcher of gemm_run picks an entry per
 * shape class.  Tiling and autotuning by shape: "矩阵乘法优化可视化学习文档",
 * section 6 "常用优化方法总表" (Tiling, Autotuning rows).
 *
 * gemm_num_configs: number of entries.
 * gemm_config_name: static text naming entry `config_id` (NULL if out of range).
 * gemm_select_config: the entry gemm_run would use for this problem with
 *                16-byte aligned operand lines, or a negative gemm_status_t
 *                if the arguments are invalid.  Entries whose kernels load
 *                operands straight into LDS ("large_dma...", and the 8-bit
 *                "i8_large_dma..." and "fp8_large_dma8...") accept only
 *                16-byte aligned operand lines, and "i8_large_dma_..." (the
 *                four-wave 16x16x64 one) only K-contiguous operands (A
 *                row-major and B column-major as the kernels see them: a
 *                column-major D swaps and flips them): with other operands
 *                gemm_run runs the register-staged 256x256 entry of the
 *                input type instead, and gemm_run_config forced to such an
 *                entry returns GEMM_ERR_INVALID_CONFIG.
 */
int gemm_num_configs(void);
const char *gemm_config_name(int config_id);
int gemm_select_config(int64_t M, int64_t N, int64_t K, int layoutA, int layoutB,
                       int in_dtype, int acc_dtype, int out_dtype);

/*
 * gemm_run with the tile-table entry forced to `config_id` (same arguments,
 * same validation, same results up to summation order).  For tests and
 * benchmarks that must reach every entry.  GEMM_ERR_INVALID_CONFIG if the
 * entry does not exist.
 */
int gemm_run_config(int config_id,
                    int64_t M, int64_t N, int64_t K,
                    const void *A, int64_t lda, int layoutA,
                    const void *B, int64_t ldb, int layoutB,
                    const void *C, int64_t ldc,
                    void *D, int64_t ldd,
                    int in_dtype, int acc_dtype, int out_dtype,
                    int satf, void *stream);

/*
 * Host-only argument check of gemm_run (no HIP call, no device needed):
 * returns GEMM_OK or the error gemm_run would return before enqueuing, except
 * the int8 satf limit on K, which depends on satf.
 */
int gemm_validate(int64_t M, int64_t N, int64_t K,
                  const void *A, int64_t lda, int layoutA,
                  const void *B, int64_t ldb, int layoutB,
                  const void *C, int64_t ldc,
                  const void *D, int64_t ldd,
                  int in_dtype, int acc_dtype, int out_dtype);

/* ===================================================== extended epilogue
 *
 * D = act( alpha * (A x B) + beta * C + bias ), rounded once to out_dtype,
 * then satf; C and D each row- or column-major.
 *
 * Sources: "矩阵乘法优化可视化学习文档", section 6 "常用优化方法总表"
 * (Epilogue fusion row: bias, activation and scale applied before the
 * write-back) and section 8 (bias/activation fused at the final store, and
 * the check that the fused result matches the unfused reference); the
 * accumulator load/store layouts mem_row_major / mem_col_major of
 * "CUDA算子优化(5)：WMMA矩阵乘法", section "WMMA API解释" items (3) and (4).
 *
 * Readings (the pages name bias, activation and scale but fix none of them):
 *  - scale is the usual pair alpha (on the product) and beta (on C); with
 *    beta == 0, C is not read (it may hold anything, NaN included);
 *  - bias holds one fp32 value per column j of D, added after the scaling;
 *  - GEMM_ACT_RELU is max(x, 0) with NaN kept and -0 -> +0; GEMM_ACT_GELU is
 *    x * Phi(x) = x/2 * (1 + erf(x / sqrt 2)), with GELU(+Inf) = +Inf and
 *    GELU(-Inf) = 0;
 *  - everything between the product and the final rounding is fp32; GELU
 *    evaluates erfc by Abramowitz & Stegun formula 7.1.26 (absolute error
 *    <= 1.5e-7), i.e. GELU to within about 2.2e-7 * max(1, |x|).
 */
typedef enum {
    GEMM_ACT_NONE = 0,
    GEMM_ACT_RELU = 1,
    GEMM_ACT_GELU = 2
} gemm_activation_t;

typedef struct {
    float alpha;          /* scale of A x B (1.0f: none)                       */
    float beta;           /* scale of C (1.0f: none; 0.0f: C is not read)      */
    const float *bias;    /* device pointer to N fp32 values, or NULL          */
    int activation;       /* gemm_activation_t                                 */
    int layoutC;          /* gemm_layout_t of C: row-major C(i,j) = C[i*ldc+j],
                             column-major C(i,j) = C[j*ldc+i]                  */
    int layoutD;          /* gemm_layout_t of D, same convention               */
} gemm_epilogue_t;

/*
 * gemm_run with the extended epilogue.  `epi` == NULL, or
 * {1, 1, NULL, GEMM_ACT_NONE, GEMM_ROW_MAJOR, GEMM_ROW_MAJOR}, is exactly
 * gemm_run (bit-identical results).  Other arguments as for gemm_run, except:
 *   ldc, ldd     >= N for a row-major matrix, >= M for a column-major one.
 *   C == D       (in place) needs ldc == ldd and layoutC == layoutD.
 *   bias         N fp32 values on the device; must not overlap D.
 * Errors, in addition to gemm_run's: an activation outside gemm_activation_t,
 * or int8 inputs with anything but the plain epilogue (alpha = 1, beta 1 or
 * 0, no bias, no activation; C/D layouts are fine) -> GEMM_ERR_UNSUPPORTED; layoutC / layoutD not a gemm_layout_t ->
 * GEMM_ERR_INVALID_LAYOUT; bias overlapping D, or C == D with different
 * layouts or leading dimensions -> GEMM_ERR_ALIASING.
 *
 * Speed: a column-major D runs the row-major kernels on D^T = B^T x A^T (the
 * operands swap roles, no data moves); C in the other layout than D, and
 * a bias pointer that is not 16-byte aligned, take the element-wise store
 * path of edge tiles.  With an fp32 D (leading dimensions of C and D
 * multiples of 4, 16-byte aligned C, D and bias) and K a multiple of the
 * tile's K step, the register-staged entries apply the whole epilogue
 * from registers; other calls stage each tile through LDS first.  GELU
 * costs about 20 vector instructions per output element.
 */
int gemm_run_ex(int64_t M, int64_t N, int64_t K,
                const void *A, int64_t lda, int layoutA,
                const void *B, int64_t ldb, int layoutB,
                const void *C, int64_t ldc,
                void *D, int64_t ldd,
                int in_dtype, int acc_dtype, int out_dtype,
                int satf, const gemm_epilogue_t *epi, void *stream);

/* gemm_run_ex with the tile-table entry forced (see gemm_run_config). */
int gemm_run_ex_config(int config_id,
                       int64_t M, int64_t N, int64_t K,
                       const void *A, int64_t lda, int layoutA,
                       const void *B, int64_t ldb, int layoutB,
                       const void *C, int64_t ldc,
                       void *D, int64_t ldd,
                       int in_dtype, int acc_dtype, int out_dtype,
                       int satf, const gemm_epilogue_t *epi, void *stream);

/* Host-only argument check of gemm_run_ex (see gemm_validate). */
int gemm_validate_ex(int64_t M, int64_t N, int64_t K,
                     const void *A, int64_t lda, int layoutA,
                     const void *B, int64_t ldb, int layoutB,
                     const void *C, int64_t ldc,
                     const void *D, int64_t ldd,
                     int in_dtype, int acc_dtype, int out_dtype,
                     const gemm_epilogue_t *epi);

/* ============================================================ autotuning
 *
 * Runtime search over the tile-shape table for one problem signature,
 * cached.  Source: "矩阵乘法优化可视化学习文档", section 6 "常用优化方法总表"
 * (Autotuning row: the best tile differs with M/N/K, dtype and GPU, and is
 * found by search) and section 8 (Autotune: one kernel timed over several
 * block sizes, the fastest kept).
 *
 * gemm_autotune runs the call once per table entry (one untimed run, then
 * `reps` timed runs, clamped to [1, 100]; the minimum counts; an entry more
 * than 2x slower than the best so far stops early), records the fastest
 * entry for the signature (M, N, K, layouts, dtypes, current device; a
 * column-major D is keyed as its transpose, which is what runs), writes it to
 * *config_out (if not NULL; -1 for an empty problem) and leaves D holding the
 * chosen entry's result.  From then on gemm_run / gemm_run_ex with that
 * signature use the recorded entry (gemm_select_config still reports the
 * static choice).  The call synchronises `stream` (HIP events), so it does
 * not belong in a timed region or a graph capture.
 * Arguments and errors as gemm_run_ex, plus: an in-place update (C == D with
 * beta != 0) -> GEMM_ERR_ALIASING, since every candidate run would apply it.
 * The cache is process-wide and guarded by a mutex.
 *
 * gemm_autotune_lookup: the recorded entry for a signature, or -1.
 * gemm_autotune_clear: forget every recorded entry.
 */
int gemm_autotune(int64_t M, int64_t N, int64_t K,
                  const void *A, int64_t lda, int layoutA,
                  const void *B, int64_t ldb, int layoutB,
                  const void *C, int64_t ldc,
                  void *D, int64_t ldd,
                  int in_dtype, int acc_dtype, int out_dtype,
                  int satf, const gemm_epilogue_t *epi, int reps, int *config_out,
                  void *stream);
int gemm_autotune_lookup(int64_t M, int64_t N, int64_t K, int layoutA, int layoutB,
                         int in_dtype, int acc_dtype, int out_dtype, int layoutD);
void gemm_autotune_clear(void);

#ifdef __cplusplus
}
#endif

#endif /* LIBGEMM_H */
