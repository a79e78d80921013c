// C ABI of libgemm: argument validation, the shape-class -> tile-table
// dispatch, the split-K workspace, and the launches.  The operation and its
// arguments are documented in include/libgemm.h.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <map>
#include <mutex>
#include <utility>
#include <vector>

#include "../../include/libgemm.h"
#include "gemm_configs.hpp"
#include "gemm_validate.hpp"

using namespace libgemm;
using namespace libgemm_host;

namespace libgemm {
// Split-K reduction: D(i,j) = finish(sum over slices in slice order + C).
// int32 outputs: the slices hold int32 bit patterns, summed in 64 bits.
__global__ void __launch_bounds__(256) splitk_reduce_kernel(Params p) {
    const int64_t total = (int64_t)p.M * p.N;
    for (int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x; idx < total;
         idx += (int64_t)gridDim.x * 256) {
        const int64_t i = idx / p.N, j = idx % p.N;
        if (p.out_dtype == DT_I32) {
            const int32_t *w = reinterpret_cast<const int32_t *>(p.ws);
            int64_t s = 0;
            for (int z = 0; z < p.splits; ++z) s += w[z * total + idx];
            if (p.C)
                s += reinterpret_cast<const int32_t *>(p.C)[p.c_col ? j * p.ldc + i
                                                                    : i * p.ldc + j];
            reinterpret_cast<int32_t *>(p.D)[i * p.ldd + j] = to_int32(s, p.satf);
        } else {
            float s = 0.0f;
            for (int z = 0; z < p.splits; ++z) s += p.ws[z * total + idx];
            finish_store(p, i, j, s);
        }
    }
}

// Copy `rows` lines of `cols` elements from lines `ld_src` apart to lines
// `ld_dst` apart (the operand repack of unaligned calls; the destination's
// padding elements are left as they are: no stored output reads them).
template <typename T>
__global__ void __launch_bounds__(256) repack_lines_kernel(const T *src, int64_t ld_src, T *dst,
                                                           int64_t ld_dst, int64_t rows,
                                                           int64_t cols) {
    for (int64_t r = blockIdx.x; r < rows; r += gridDim.x) {
        const T *s = src + r * ld_src;
        T *d = dst + r * ld_dst;
        for (int64_t c = threadIdx.x; c < cols; c += 256) d[c] = s[c];
    }
}

}  // namespace libgemm

namespace {

struct Entry {
    const char *name;
    int BM, BN, BK;
    int split_k;  // 1: this entry may split K across workgroups
    int klass;    // input class: 0 = fp16/bf16, 1 = int8, 2 = OCP fp8
    launch_fn launch;
};

const Entry kTable[] = {
    {"large_256x256x64_w2x2_mfma32x32x16", CfgLarge::BM, CfgLarge::BN, CfgLarge::BK, 0, 0,
     launch_large},
    {"medium_128x128x64_w2x2_mfma32x32x16", CfgMedium::BM, CfgMedium::BN, CfgMedium::BK, 0, 0,
     launch_medium},
    {"small_64x64x64_w2x2_mfma32x32x16", CfgSmall::BM, CfgSmall::BN, CfgSmall::BK, 0, 0,
     launch_small},
    {"skinny_16x128x128_w1x4_mfma16x16x32_splitk", CfgSkinny::BM, CfgSkinny::BN, CfgSkinny::BK, 1,
     0, launch_skinny},
    {"large8_256x256x64_w2x4_mfma32x32x16", CfgLarge8::BM, CfgLarge8::BN, CfgLarge8::BK, 0, 0,
     launch_large8},
    {"i8_large8_256x256x128_w2x4_mfma32x32x32", CfgLarge8I8::BM, CfgLarge8I8::BN, CfgLarge8I8::BK,
     0, 1, launch_large8_i8},
    {"i8_medium_128x128x128_w2x2_mfma32x32x32", CfgMediumI8::BM, CfgMediumI8::BN, CfgMediumI8::BK,
     0, 1, launch_medium_i8},
    {"i8_small_64x64x128_w2x2_mfma32x32x32", CfgSmallI8::BM, CfgSmallI8::BN, CfgSmallI8::BK, 0, 1,
     launch_small_i8},
    {"i8_skinny_16x128x256_w1x4_mfma16x16x64_splitk", CfgSkinnyI8::BM, CfgSkinnyI8::BN,
     CfgSkinnyI8::BK, 1, 1, launch_skinny_i8},
    {"fp8_large_256x256x128_w2x2_mfma32x32x64", CfgLargeF8::BM, CfgLargeF8::BN,
     CfgLargeF8::BK, 0, 2, launch_large_fp8},
    {"fp8_medium_128x128x128_w2x2_mfma32x32x64", CfgMediumF8::BM, CfgMediumF8::BN,
     CfgMediumF8::BK, 0, 2, launch_medium_fp8},
    {"fp8_small_64x64x128_w2x2_mfma32x32x64", CfgSmallF8::BM, CfgSmallF8::BN, CfgSmallF8::BK, 0,
     2, launch_small_fp8},
    {"fp8_skinny_16x128x256_w1x4_mfma16x16x128_splitk", CfgSkinnyF8::BM, CfgSkinnyF8::BN,
     CfgSkinnyF8::BK, 1, 2, launch_skinny_fp8},
    {"large_dma_256x256x64_w2x2_mfma32x32x16", CfgLargeDma::BM, CfgLargeDma::BN, CfgLargeDma::BK,
     0, 0, launch_large_dma},
    {"tiny_32x32x64_w1x1_mfma32x32x16", CfgTiny::BM, CfgTiny::BN, CfgTiny::BK, 0, 0, launch_tiny},
    {"large_dma_256x256x64_w2x2_mfma16x16x32", CfgLargeDma16::BM, CfgLargeDma16::BN,
     CfgLargeDma16::BK, 0, 0, launch_large_dma16},
    {"large_dma8_256x256x64_w2x4_mfma16x16x32", CfgLargeDma8_16::BM, CfgLargeDma8_16::BN,
     CfgLargeDma8_16::BK, 0, 0, launch_large_dma8_16},
    {"i8_large_dma8_256x256x128_w2x4_mfma32x32x32", CfgLargeDma8I8::BM, CfgLargeDma8I8::BN,
     CfgLargeDma8I8::BK, 0, 1, launch_large_dma8_i8},
    {"fp8_large_dma8_256x256x128_w2x4_mfma32x32x64", CfgLargeDma8F8::BM, CfgLargeDma8F8::BN,
     CfgLargeDma8F8::BK, 0, 2, launch_large_dma8_fp8},
    {"i8_large_dma_256x256x128_w2x2_mfma16x16x64", CfgLargeDmaI8_16::BM, CfgLargeDmaI8_16::BN,
     CfgLargeDmaI8_16::BK, 0, 1, launch_large_dma16_i8},
};
constexpr int kNumConfigs = sizeof(kTable) / sizeof(kTable[0]);
enum { CFG_LARGE = 0, CFG_MEDIUM = 1, CFG_SMALL = 2, CFG_SKINNY = 3, CFG_LARGE8 = 4,
       CFG_I8_LARGE8 = 5, CFG_I8_MEDIUM = 6, CFG_I8_SMALL = 7, CFG_I8_SKINNY = 8,
       CFG_F8_LARGE = 9, CFG_F8_MEDIUM = 10, CFG_F8_SMALL = 11, CFG_F8_SKINNY = 12,
       CFG_LARGE_DMA = 13, CFG_TINY = 14, CFG_LARGE_DMA16 = 15, CFG_LARGE_DMA8_16 = 16,
       CFG_I8_LARGE_DMA8 = 17, CFG_F8_LARGE_DMA8 = 18, CFG_I8_LARGE_DMA16 = 19 };

// Entries whose kernels load operands straight into LDS: 16-byte aligned
// operands only (vec_ok); others run the entry of the same tile shape
// with register-staged loads.
bool needs_vec(int id) {
    return id == CFG_LARGE_DMA || id == CFG_LARGE_DMA16 || id == CFG_LARGE_DMA8_16 ||
           id == CFG_I8_LARGE_DMA8 || id == CFG_F8_LARGE_DMA8 || id == CFG_I8_LARGE_DMA16;
}
// Entries for K-contiguous operands only (as the kernels see them: row-major
// A, column-major B).
bool needs_kc(int id) { return id == CFG_I8_LARGE_DMA16; }
// the register-staged large tile of each input class
int class_large(int klass) {
    return klass == 1 ? CFG_I8_LARGE8 : klass == 2 ? CFG_F8_LARGE : CFG_LARGE8;
}


// Compute units and XCDs of the current device, read once per device from
// its attributes (MI355X: 256 CUs in 8 XCDs, which is also the answer when no
// device can be queried, e.g. for gemm_select_config on a host without GPU).
struct Topology {
    int cus, xcds;
};
constexpr int kMaxDevices = 64;
constexpr Topology kDefaultTopology = {256, 8};
std::mutex g_topo_mutex;
Topology g_topo[kMaxDevices];
bool g_topo_known[kMaxDevices];

Topology topology() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
        return kDefaultTopology;
    std::lock_guard<std::mutex> lock(g_topo_mutex);
    if (!g_topo_known[dev]) {
        Topology t = kDefaultTopology;
        int v = 0;
        if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess &&
            v > 0)
            t.cus = v;
        v = 0;
        if (hipDeviceGetAttribute(&v, hipDeviceAttributeNumberOfXccs, dev) == hipSuccess && v > 0)
            t.xcds = v;
        g_topo[dev] = t;
        g_topo_known[dev] = true;
    }
    return g_topo[dev];
}

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

int select_config(int64_t M, int64_t N, int64_t K, int klass, int cus) {
    (void)K;
    // the same shape classes for every input class; entries per class
    // (skinny, large, medium, small, tiny; the 8-bit classes have no tiny tile)
    static const int kByClass[3][5] = {
        {CFG_SKINNY, CFG_LARGE8, CFG_MEDIUM, CFG_SMALL, CFG_TINY},
        {CFG_I8_SKINNY, CFG_I8_LARGE8, CFG_I8_MEDIUM, CFG_I8_SMALL, CFG_I8_SMALL},
        {CFG_F8_SKINNY, CFG_F8_LARGE, CFG_F8_MEDIUM, CFG_F8_SMALL, CFG_F8_SMALL}};
    const int *e = kByClass[klass];
    if (M <= CfgSkinny::BM) return e[0];
    const int64_t t_large = cdiv(M, CfgLarge::BM) * cdiv(N, CfgLarge::BN);
    if (t_large >= 3 * cus / 4) return e[1];
    const int64_t t_medium = cdiv(M, CfgMedium::BM) * cdiv(N, CfgMedium::BN);
    if (t_medium >= cus / 2) return e[2];
    const int64_t t_small = cdiv(M, CfgSmall::BM) * cdiv(N, CfgSmall::BN);
    if (t_small >= cus / 2) return e[3];
    return e[4];
}

// The dispatcher's large tiles.  16-bit: with both operands K-contiguous (A
// row-major, B column-major) and 16-byte aligned, the LDS-DMA kernel with the
// 16x16x32 MFMA (measured 6-8% faster at 4096^3: that MFMA sustains a higher
// clock under the power limit); an N- or M-contiguous operand would need
// transposed LDS reads, which cost more than the register-staged transpose
// of the eight-wave tile.  int8: the same four-wave shape with the 16x16x64
// MFMA for K-contiguous aligned operands and whole K-tiles (4096^3 ~10%
// faster than the eight-wave register-staged tile; its ragged-K kernel
// spills, so a ragged K keeps the register-staged tile, as do the other
// layouts).  fp8 with 16-byte aligned lines: the eight-wave LDS-DMA tile in
// every layout (4096^3: K-contiguous ~6% faster than the four-wave
// register-staged tile, on par at K = 4100; M- or N-contiguous operands
// 83-108 us against 140-176 us on the 128x128 tile, which they took because
// the four-wave tile spills with its transposing loads).
int refine_large(int id, bool aligned, int layoutA, int layoutB, int64_t K) {
    const bool kc = layoutA == GEMM_ROW_MAJOR && layoutB == GEMM_COL_MAJOR;
    if (id == CFG_LARGE8 && aligned && kc) return CFG_LARGE_DMA16;
    if (id == CFG_I8_LARGE8 && aligned && kc && K % CfgLargeDmaI8_16::BK == 0)
        return CFG_I8_LARGE_DMA16;
    if (id == CFG_F8_LARGE && aligned) return CFG_F8_LARGE_DMA8;
    return id;
}

// Autotuned choices: problem signature (as the kernels see it, after a
// column-major D has been turned into D^T) -> table entry.  Process-wide.
struct TuneKey {
    int64_t M, N, K;
    int layoutA, layoutB, in_dtype, acc_dtype, out_dtype, device;
    bool operator<(const TuneKey &o) const {
        const int64_t a[9] = {M, N, K, layoutA, layoutB, in_dtype, acc_dtype, out_dtype, device};
        const int64_t b[9] = {o.M, o.N, o.K, o.layoutA, o.layoutB, o.in_dtype, o.acc_dtype,
                              o.out_dtype, o.device};
        for (int i = 0; i < 9; ++i)
            if (a[i] != b[i]) return a[i] < b[i];
        return false;
    }
};
std::mutex g_tune_mutex;
std::map<TuneKey, int> g_tune;

int current_device() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return -1;
    return dev;
}

int tuned_config(const TuneKey &k) {
    std::lock_guard<std::mutex> lock(g_tune_mutex);
    auto it = g_tune.find(k);
    return it == g_tune.end() ? -1 : it->second;
}

// Split-K workspace, one per (device, stream), grown on demand with
// hipMalloc.  g_ws_mutex is held by a call from the moment it takes the buffer
// until both of its launches are enqueued, so the work of two calls on one
// stream is enqueued one call after the other and each reads only its own
// partial sums (stream order).  A buffer that is outgrown may still be in use
// by work enqueued earlier, so it is never freed: it moves to g_ws_retired
// and, like the current buffers, is kept until the process exits.
std::mutex g_ws_mutex;
std::map<std::pair<int, hipStream_t>, std::pair<float *, size_t>> g_ws;
std::vector<float *> g_ws_retired;

// The caller holds g_ws_mutex.
hipError_t workspace_locked(hipStream_t stream, size_t bytes, float **out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    auto &slot = g_ws[std::make_pair(dev, stream)];
    if (slot.second < bytes) {
        // grow at least 2x, so a sequence of growing calls retires few buffers
        const size_t want = bytes > 2 * slot.second ? bytes : 2 * slot.second;
        void *ptr = nullptr;
        e = hipMalloc(&ptr, want);
        if (e != hipSuccess) return e;
        if (slot.first) g_ws_retired.push_back(slot.first);
        slot.first = static_cast<float *>(ptr);
        slot.second = want;
    }
    *out = slot.first;
    return hipSuccess;
}

// Scratch of the allocation-free entry point (gemm_run_noalloc): split-K
// partial sums in a device array of fixed size, one copy per device, held
// until the process ends.  Host code never uses the array's name as an
// address: on each device, the first gemm_run_noalloc call (with that device
// current) looks up the array's device address with hipGetSymbolAddress and
// keeps it; kernels get that address.
constexpr size_t kScratchBytes = (size_t)32 << 20;
static __device__ __align__(256) float scratch[kScratchBytes / sizeof(float)];
std::mutex g_scratch_mutex;
float *g_scratch_ptr[kMaxDevices];

hipError_t scratch_address(float **out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch_ptr[dev]) {
        void *ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!ptr) return hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = static_cast<float *>(ptr);
    }
    *out = g_scratch_ptr[dev];
    return hipSuccess;
}

// Where run() takes the split-K workspace from.
enum WorkspaceMode { WS_LIBRARY = 0, WS_STATIC_SCRATCH = 1 };

// The copy of one operand into the workspace with lines of whole 16-byte
// units (bytes == 0: no copy).  outer lines of inner elements of isz bytes.
struct Repack {
    int64_t outer = 0, inner = 0, ld = 0;  // ld: the copy's leading dimension
    size_t bytes = 0;                      // workspace bytes (256-byte multiple)
    int64_t rng = 0;                       // the copy's extent, rounded up to 16 bytes
};

Repack plan_repack(const void *X, int64_t ld, int64_t outer, int64_t inner, int isz) {
    Repack r;
    if ((uintptr_t)X % 16 == 0 && (ld * isz) % 16 == 0) return r;  // already aligned
    const int64_t per = 16 / isz;  // elements per 16 bytes
    r.outer = outer;
    r.inner = inner;
    r.ld = (inner + per - 1) / per * per;
    r.rng = ((outer - 1) * r.ld + inner) * isz;
    r.rng = (r.rng + 15) & ~(int64_t)15;
    r.bytes = ((size_t)(outer * r.ld * isz) + 255) & ~(size_t)255;
    return r;
}

hipError_t launch_repack(const void *src, int64_t ld_src, void *dst, const Repack &r, int isz,
                         hipStream_t s) {
    const int cus = topology().cus;
    const int64_t blocks = r.outer < 8 * (int64_t)cus ? r.outer : 8 * (int64_t)cus;
    const dim3 grid((unsigned)blocks), block(256);
    if (isz == 2) {
        const uint16_t *sp = static_cast<const uint16_t *>(src);
        uint16_t *dp = static_cast<uint16_t *>(dst);
        int64_t lds = ld_src, ldd = r.ld, rows = r.outer, cols = r.inner;
        void *args[] = {&sp, &lds, &dp, &ldd, &rows, &cols};
        return hipLaunchKernel(reinterpret_cast<const void *>(repack_lines_kernel<uint16_t>), grid,
                               block, args, 0, s);
    }
    const uint8_t *sp = static_cast<const uint8_t *>(src);
    uint8_t *dp = static_cast<uint8_t *>(dst);
    int64_t lds = ld_src, ldd = r.ld, rows = r.outer, cols = r.inner;
    void *args[] = {&sp, &lds, &dp, &ldd, &rows, &cols};
    return hipLaunchKernel(reinterpret_cast<const void *>(repack_lines_kernel<uint8_t>), grid,
                           block, args, 0, s);
}

int run(int config_id, int64_t M, int64_t N, int64_t K, const void *A, int64_t lda,
        int layoutA, const void *B, int64_t ldb, int layoutB, const void *C, int64_t ldc,
        void *D, int64_t ldd, int in_dtype, int acc_dtype, int out_dtype, int satf,
        const gemm_epilogue_t *epi_arg, void *stream_handle, int ws_mode = WS_LIBRARY) {
    int st = validate(M, N, K, A, lda, layoutA, B, ldb, layoutB, C, ldc, D, ldd, in_dtype,
                      acc_dtype, out_dtype, epi_arg, satf);
    if (st != GEMM_OK) return st;
    const int klass = input_class(in_dtype);
    if (config_id >= kNumConfigs || (config_id >= 0 && kTable[config_id].klass != klass))
        return GEMM_ERR_INVALID_CONFIG;
    if (M == 0 || N == 0) return GEMM_OK;
    const gemm_epilogue_t epi = epi_arg ? *epi_arg : kPlainEpilogue;
    if (epi.beta == 0.0f) C = nullptr;  // beta == 0: C is not read
    int layoutC = epi.layoutC;
    bool bias_rows = false;
    if (epi.layoutD == GEMM_COL_MAJOR) {
        // A column-major D is the row-major N x M matrix D^T = B^T x A^T: swap
        // the operands (each keeps its memory, its layout flag flips), M and
        // N, and index the bias by row
        const void *t = A;
        A = B;
        B = t;
        const int64_t tl = lda;
        lda = ldb;
        ldb = tl;
        const int la = layoutA;
        layoutA = layoutB == GEMM_ROW_MAJOR ? GEMM_COL_MAJOR : GEMM_ROW_MAJOR;
        layoutB = la == GEMM_ROW_MAJOR ? GEMM_COL_MAJOR : GEMM_ROW_MAJOR;
        const int64_t tm = M;
        M = N;
        N = tm;
        layoutC = layoutC == GEMM_ROW_MAJOR ? GEMM_COL_MAJOR : GEMM_ROW_MAJOR;
        bias_rows = true;
    }
    const Topology topo = topology();
    int id = config_id;
    bool auto_choice = false;  // the static dispatcher's pick (not forced, not autotuned)
    if (id < 0) {
        const TuneKey key{M, N, K, layoutA, layoutB, in_dtype, acc_dtype, out_dtype,
                          current_device()};
        id = tuned_config(key);
        if (id < 0) {
            id = select_config(M, N, K, klass, topo.cus);
            auto_choice = true;
        }
    }
    hipStream_t stream = static_cast<hipStream_t>(stream_handle);

    Params p{};
    p.A = static_cast<const uint16_t *>(A);
    p.B = static_cast<const uint16_t *>(B);
    p.C = C;
    p.D = D;
    p.ws = nullptr;
    p.lda = lda;
    p.ldb = ldb;
    p.ldc = C ? ldc : 0;
    p.ldd = ldd;
    p.M = (int)M;
    p.N = (int)N;
    p.K = (int)K;
    p.out_dtype = out_dtype;
    p.satf = satf ? 1 : 0;
    p.c_col = (C && layoutC == GEMM_COL_MAJOR) ? 1 : 0;
    p.alpha = epi.alpha;
    p.beta = epi.beta;
    p.bias = epi.bias;
    p.bias_rows = bias_rows ? 1 : 0;
    p.act = epi.activation;
    p.epi = (epi.alpha != 1.0f || (C && epi.beta != 1.0f) || epi.bias ||
             epi.activation != GEMM_ACT_NONE || p.c_col) ? 1 : 0;
    // Vector path: 16-byte aligned operands (lines a multiple of 16 bytes)
    // whose extents, rounded up to 16 bytes, fit a 32-bit buffer range
    const int isz = in_size(in_dtype);
    const int64_t a_ext =
        (layoutA == GEMM_ROW_MAJOR ? (M - 1) * lda + K : (K - 1) * lda + M) * isz;
    const int64_t b_ext =
        (layoutB == GEMM_ROW_MAJOR ? (K - 1) * ldb + N : (N - 1) * ldb + K) * isz;
    const int64_t a_rng = (a_ext + 15) & ~(int64_t)15, b_rng = (b_ext + 15) & ~(int64_t)15;
    int64_t a_rng_used = a_rng, b_rng_used = b_rng;
    p.vec_ok = K > 0 && ((uintptr_t)A % 16 == 0) && ((uintptr_t)B % 16 == 0) &&
               ((lda * isz) % 16 == 0) && ((ldb * isz) % 16 == 0) &&
               a_rng < ((int64_t)1 << 32) - 16 && b_rng < ((int64_t)1 << 32) - 16;
    // Large calls whose operands miss the vector path only by alignment copy
    // the offending operand(s) into the library workspace with lines of
    // whole 16-byte units first (a line copy costs far less than the
    // element-wise loads: 4096^3 fp16 with lda = 4097 ~600 us unpacked).  The
    // call without allocation (gemm_run_noalloc) keeps the element path.
    Repack rp_a, rp_b;
    if (!p.vec_ok && ws_mode == WS_LIBRARY && K > 0 && M * N * K >= ((int64_t)1 << 30)) {
        rp_a = plan_repack(A, lda, layoutA == GEMM_ROW_MAJOR ? M : K,
                           layoutA == GEMM_ROW_MAJOR ? K : M, isz);
        rp_b = plan_repack(B, ldb, layoutB == GEMM_ROW_MAJOR ? K : N,
                           layoutB == GEMM_ROW_MAJOR ? N : K, isz);
        const int64_t a2 = rp_a.bytes ? rp_a.rng : a_rng, b2 = rp_b.bytes ? rp_b.rng : b_rng;
        const bool a_al = rp_a.bytes || (((uintptr_t)A % 16 == 0) && ((lda * isz) % 16 == 0));
        const bool b_al = rp_b.bytes || (((uintptr_t)B % 16 == 0) && ((ldb * isz) % 16 == 0));
        if (a_al && b_al && a2 < ((int64_t)1 << 32) - 16 && b2 < ((int64_t)1 << 32) - 16) {
            p.vec_ok = 1;
            a_rng_used = a2;
            b_rng_used = b2;
        } else {
            rp_a = Repack{};
            rp_b = Repack{};
        }
    }
    p.a_bytes = p.vec_ok ? (uint32_t)a_rng_used : 0u;
    p.b_bytes = p.vec_ok ? (uint32_t)b_rng_used : 0u;
    const bool kc_ops = layoutA == GEMM_ROW_MAJOR && layoutB == GEMM_COL_MAJOR;
    if ((needs_vec(id) && !p.vec_ok) || (needs_kc(id) && !kc_ops)) {
        // a forced entry that cannot run these operands is an error; the
        // dispatcher's choice falls back to the register-staged large tile
        if (config_id >= 0) return GEMM_ERR_INVALID_CONFIG;
        id = class_large(klass);
    }
    if (auto_choice) id = refine_large(id, p.vec_ok != 0, layoutA, layoutB, K);
    const Entry &E = kTable[id];
    const int osz = out_size(out_dtype);
    // register epilogue (vector C, D and bias access): aligned row-major C and D
    p.cd_vec = ((uintptr_t)D % (4 * osz) == 0) && (ldd % 4 == 0) &&
               (!C || (((uintptr_t)C % (4 * osz) == 0) && (ldc % 4 == 0) && !p.c_col)) &&
               (!p.bias || p.bias_rows || (uintptr_t)p.bias % 16 == 0);
    p.tiles_m = (int)cdiv(M, E.BM);
    p.tiles_n = (int)cdiv(N, E.BN);
    const int64_t tiles = (int64_t)p.tiles_m * p.tiles_n;
    if (tiles > 0x7fffffff) return GEMM_ERR_INVALID_DIM;
    // Raster groups of 4 tile-rows per XCD keep the L2 fills low.  When each
    // CU runs several 256x256 tiles with a short K loop, D's stores and the B
    // panels' refills share the memory system with the K loop: groups of 2
    // tile-rows whose starting columns are staggered by group (skew) halve
    // the B refills of row order and keep the XCDs on different column bands
    // (16384^2 x 1024: 3-4% faster than row order for fp16, 5% for int8;
    // unstaggered groups of 2 to 8 rows were 8-40% slower than row order,
    // as every XCD then streams the same narrow column band).  At 8192^3 and
    // at one tile per CU the stagger changed nothing measurable.
    const bool short_multi = E.BM == 256 && tiles > topo.cus && K <= 2048;
    p.group_m = short_multi ? 2 : 4;
    p.skew = short_multi ? 1 : 0;
    p.xcds = topo.xcds;

    // K slices: enough workgroups for 4 per CU, each slice >= 8 K-tiles
    int splits = 1;
    if (E.split_k && K > 0) {
        const int64_t want = cdiv(4 * (int64_t)topo.cus, tiles);
        const int64_t most = cdiv(K, (int64_t)E.BK * 8);
        splits = (int)(want < most ? want : most);
        if (splits < 1) splits = 1;
    }
    int64_t kps = cdiv(cdiv(K > 0 ? K : 1, splits), E.BK) * E.BK;
    splits = (int)cdiv(K > 0 ? K : 1, kps);
    p.splits = splits;
    p.k_per_split = (int)kps;

    const int akc = layoutA == GEMM_ROW_MAJOR;
    const int bkc = layoutB == GEMM_COL_MAJOR;
    dim3 grid((unsigned)tiles, 1, (unsigned)splits);
    // the launcher's variant flag: bf16 among the 16-bit inputs, E5M2 among fp8
    const int variant = (in_dtype == GEMM_BF16 || in_dtype == GEMM_FP8_E5M2) ? 1 : 0;
    const bool repack = rp_a.bytes || rp_b.bytes;
    if (splits == 1 && !repack)
        return E.launch(p, variant, akc, bkc, grid, stream) == hipSuccess ? GEMM_OK : GEMM_ERR_HIP;

    // Workspace: repacked operands, then the split-K slices.  The lock is
    // held until every launch of the call is enqueued, so the call's
    // launches stay in one piece in the stream's order.
    const size_t ws_split = splits > 1 ? (size_t)splits * (size_t)M * (size_t)N * sizeof(float) : 0;
    const size_t ws_bytes = rp_a.bytes + rp_b.bytes + ws_split;
    std::unique_lock<std::mutex> ws_lock;
    char *ws = nullptr;
    if (ws_mode == WS_STATIC_SCRATCH) {
        if (ws_bytes > kScratchBytes) return GEMM_ERR_SCRATCH_TOO_SMALL;
        float *w = nullptr;
        if (scratch_address(&w) != hipSuccess) return GEMM_ERR_HIP;
        ws = reinterpret_cast<char *>(w);
    } else {
        ws_lock = std::unique_lock<std::mutex>(g_ws_mutex);
        float *w = nullptr;
        if (workspace_locked(stream, ws_bytes, &w) != hipSuccess) return GEMM_ERR_HIP;
        ws = reinterpret_cast<char *>(w);
    }
    if (rp_a.bytes) {
        if (launch_repack(A, lda, ws, rp_a, isz, stream) != hipSuccess) return GEMM_ERR_HIP;
        p.A = reinterpret_cast<const uint16_t *>(ws);
        p.lda = rp_a.ld;
    }
    if (rp_b.bytes) {
        char *dst = ws + rp_a.bytes;
        if (launch_repack(B, ldb, dst, rp_b, isz, stream) != hipSuccess) return GEMM_ERR_HIP;
        p.B = reinterpret_cast<const uint16_t *>(dst);
        p.ldb = rp_b.ld;
    }
    p.ws = reinterpret_cast<float *>(ws + rp_a.bytes + rp_b.bytes);
    if (splits == 1)
        return E.launch(p, variant, akc, bkc, grid, stream) == hipSuccess ? GEMM_OK : GEMM_ERR_HIP;

    // split-K: slice kernel into the workspace, then the reduction into D
    if (E.launch(p, variant, akc, bkc, grid, stream) != hipSuccess) return GEMM_ERR_HIP;
    const int64_t total = M * N;
    int64_t blocks = cdiv(total, 256);
    if (blocks > 8 * (int64_t)topo.cus) blocks = 8 * (int64_t)topo.cus;
    if (launch_params(splitk_reduce_kernel, dim3((unsigned)blocks), dim3(256), p, stream) !=
        hipSuccess)
        return GEMM_ERR_HIP;
    return GEMM_OK;
}

// The problem signature the kernels see (a column-major D becomes D^T).
TuneKey tune_key(int64_t M, int64_t N, int64_t K, int layoutA, int layoutB, int in_dtype,
                 int acc_dtype, int out_dtype, int layoutD) {
    if (layoutD == GEMM_COL_MAJOR) {
        const int la = layoutA;
        layoutA = layoutB == GEMM_ROW_MAJOR ? GEMM_COL_MAJOR : GEMM_ROW_MAJOR;
        layoutB = la == GEMM_ROW_MAJOR ? GEMM_COL_MAJOR : GEMM_ROW_MAJOR;
        const int64_t t = M;
        M = N;
        N = t;
    }
    return TuneKey{M, N, K, layoutA, layoutB, in_dtype, acc_dtype, out_dtype, current_device()};
}

int autotune(int64_t M, int64_t N, int64_t K, const void *A, int64_t lda, int layoutA,
             const void *B, int64_t ldb, int layoutB, const void *C, int64_t ldc, void *D,
             int64_t ldd, int in_dtype, int acc_dtype, int out_dtype, int satf,
             const gemm_epilogue_t *epi, int reps, int *config_out, void *stream_handle) {
    int st = validate(M, N, K, A, lda, layoutA, B, ldb, layoutB, C, ldc, D, ldd, in_dtype,
                      acc_dtype, out_dtype, epi, satf);
    if (st != GEMM_OK) return st;
    const gemm_epilogue_t e = epi ? *epi : kPlainEpilogue;
    // every candidate runs the call: an in-place update would compound
    if (C && C == D && e.beta != 0.0f) return GEMM_ERR_ALIASING;
    if (reps < 1) reps = 1;
    if (reps > 100) reps = 100;
    if (M == 0 || N == 0) {
        if (config_out) *config_out = -1;
        return GEMM_OK;
    }
    hipStream_t stream = static_cast<hipStream_t>(stream_handle);
    hipEvent_t ev[2];
    if (hipEventCreate(&ev[0]) != hipSuccess) return GEMM_ERR_HIP;
    if (hipEventCreate(&ev[1]) != hipSuccess) {
        (void)hipEventDestroy(ev[0]);
        return GEMM_ERR_HIP;
    }
    int best = -1;
    float best_ms = 0.0f;
    st = GEMM_OK;
    for (int id = 0; id < kNumConfigs && st == GEMM_OK; ++id) {
        if (kTable[id].klass != input_class(in_dtype)) continue;
        // one untimed run, then reps timed runs; the minimum counts.  An
        // entry already 2x slower than the best on its first timed run stops.
        float cand = -1.0f;
        for (int r = 0; r <= reps && st == GEMM_OK; ++r) {
            if (hipEventRecord(ev[0], stream) != hipSuccess) { st = GEMM_ERR_HIP; break; }
            st = run(id, M, N, K, A, lda, layoutA, B, ldb, layoutB, C, ldc, D, ldd, in_dtype,
                     acc_dtype, out_dtype, satf, epi, stream_handle);
            if (st == GEMM_ERR_INVALID_CONFIG) {  // this entry cannot run these operands
                st = GEMM_OK;
                cand = -1.0f;
                break;
            }
            if (st != GEMM_OK) break;
            float ms = 0.0f;
            if (hipEventRecord(ev[1], stream) != hipSuccess ||
                hipEventSynchronize(ev[1]) != hipSuccess ||
                hipEventElapsedTime(&ms, ev[0], ev[1]) != hipSuccess) {
                st = GEMM_ERR_HIP;
                break;
            }
            if (r == 0) continue;
            if (cand < 0.0f || ms < cand) cand = ms;
            if (best >= 0 && cand > 2.0f * best_ms) break;
        }
        if (st == GEMM_OK && cand >= 0.0f && (best < 0 || cand < best_ms)) {
            best = id;
            best_ms = cand;
        }
    }
    (void)hipEventDestroy(ev[0]);
    (void)hipEventDestroy(ev[1]);
    if (st != GEMM_OK) return st;
    {
        std::lock_guard<std::mutex> lock(g_tune_mutex);
        g_tune[tune_key(M, N, K, layoutA, layoutB, in_dtype, acc_dtype, out_dtype,
                        e.layoutD)] = best;
    }
    if (config_out) *config_out = best;
    // leave D holding the chosen entry's result
    return run(best, M, N, K, A, lda, layoutA, B, ldb, layoutB, C, ldc, D, ldd, in_dtype,
               acc_dtype, out_dtype, satf, epi, stream_handle);
}

}  // namespace

extern "C" {

int gemm_autotune(int64_t M, int64_t N, int64_t K, const void *A, int64_t lda, int layoutA,
                  const void *B, int64_t ldb, int layoutB, const void *C, int64_t ldc, void *D,
                  int64_t ldd, int in_dtype, int acc_dtype, int out_dtype, int satf,
                  const gemm_epilogue_t *epi, int reps, int *config_out, void *stream) {
    return autotune(M, N, K, A, lda, layoutA, B, ldb, layoutB, C, ldc, D, ldd, in_dtype,
                    acc_dtype, out_dtype, satf, epi, reps, config_out, stream);
}

int gemm_autotune_lookup(int64_t M, int64_t N, int64_t K, int layoutA, int layoutB,
                         int in_dtype, int acc_dtype, int out_dtype, int layoutD) {
    return tuned_config(tune_key(M, N, K, layoutA, layoutB, in_dtype, acc_dtype, out_dtype,
                                 layoutD));
}

void gemm_autotune_clear(void) {
    std::lock_guard<std::mutex> lock(g_tune_mutex);
    g_tune.clear();
}

int gemm_validate(int64_t M, int64_t N, int64_t K, const void *A, int64_t lda, int layoutA,
                  const void *B, int64_t ldb, int layoutB, const void *C, int64_t ldc,
                  const void *D, int64_t ldd, int in_dtype, int acc_dtype, int out_dtype) {
    return validate(M, N, K, A, lda, layoutA, B, ldb, layoutB, C, ldc, D, ldd, in_dtype,
                    acc_dtype, out_dtype, nullptr, 0);
}

int gemm_validate_ex(int64_t M, int64_t N, int64_t K, const void *A, int64_t lda, int layoutA,
                     const void *B, int64_t ldb, int layoutB, const void *C, int64_t ldc,
                     const void *D, int64_t ldd, int in_dtype, int acc_dtype, int out_dtype,
                     const gemm_epilogue_t *epi) {
    return validate(M, N, K, A, lda, layoutA, B, ldb, layoutB, C, ldc, D, ldd, in_dtype,
                    acc_dtype, out_dtype, epi, 0);
}

int gemm_run_ex(int64_t M, int64_t N, int64_t K, const void *A, int64_t lda, int layoutA,
                const void *B, int64_t ldb, int layoutB, const void *C, int64_t ldc, void *D,
                int64_t ldd, int in_dtype, int acc_dtype, int out_dtype, int satf,
                const gemm_epilogue_t *epi, void *stream) {
    return run(-1, M, N, K, A, lda, layoutA, B, ldb, layoutB, C, ldc, D, ldd, in_dtype,
               acc_dtype, out_dtype, satf, epi, stream);
}

int gemm_run_ex_config(int config_id, int64_t M, int64_t N, int64_t K, const void *A,
                       int64_t lda, int layoutA, const void *B, int64_t ldb, int layoutB,
                       const void *C, int64_t ldc, void *D, int64_t ldd, int in_dtype,
                       int acc_dtype, int out_dtype, int satf, const gemm_epilogue_t *epi,
                       void *stream) {
    if (config_id < 0 || config_id >= kNumConfigs) return GEMM_ERR_INVALID_CONFIG;
    return run(config_id, M, N, K, A, lda, layoutA, B, ldb, layoutB, C, ldc, D, ldd, in_dtype,
               acc_dtype, out_dtype, satf, epi, stream);
}

int gemm_run(int64_t M, int64_t N, int64_t K, const void *A, int64_t lda, int layoutA,
             const void *B, int64_t ldb, int layoutB, const void *C, int64_t ldc, void *D,
             int64_t ldd, int in_dtype, int acc_dtype, int out_dtype, int satf, void *stream) {
    return run(-1, M, N, K, A, lda, layoutA, B, ldb, layoutB, C, ldc, D, ldd, in_dtype, acc_dtype,
               out_dtype, satf, nullptr, stream);
}

int gemm_run_noalloc(int64_t M, int64_t N, int64_t K, const void *A, int64_t lda, int layoutA,
                     const void *B, int64_t ldb, int layoutB, const void *C, int64_t ldc, void *D,
                     int64_t ldd, int in_dtype, int acc_dtype, int out_dtype, int satf,
                     void *stream) {
    return run(-1, M, N, K, A, lda, layoutA, B, ldb, layoutB, C, ldc, D, ldd, in_dtype, acc_dtype,
               out_dtype, satf, nullptr, stream, WS_STATIC_SCRATCH);
}

int gemm_run_config(int config_id, int64_t M, int64_t N, int64_t K, const void *A, int64_t lda,
                    int layoutA, const void *B, int64_t ldb, int layoutB, const void *C,
                    int64_t ldc, void *D, int64_t ldd, int in_dtype, int acc_dtype,
                    int out_dtype, int satf, void *stream) {
    if (config_id < 0 || config_id >= kNumConfigs) return GEMM_ERR_INVALID_CONFIG;
    return run(config_id, M, N, K, A, lda, layoutA, B, ldb, layoutB, C, ldc, D, ldd, in_dtype,
               acc_dtype, out_dtype, satf, nullptr, stream);
}

const char *gemm_status_string(int status) {
    switch (status) {
    case GEMM_OK: return "ok";
    case GEMM_ERR_INVALID_DIM: return "invalid dimension (negative or above 2^31-1)";
    case GEMM_ERR_INVALID_LD: return "leading dimension too small (or too large)";
    case GEMM_ERR_NULL_PTR: return "null pointer for a non-empty operand";
    case GEMM_ERR_UNSUPPORTED: return "unsupported dtype combination";
    case GEMM_ERR_INVALID_LAYOUT: return "layout must be GEMM_ROW_MAJOR or GEMM_COL_MAJOR";
    case GEMM_ERR_ALIASING: return "D overlaps A or B, or C partially overlaps D";
    case GEMM_ERR_HIP: return "HIP runtime error";
    case GEMM_ERR_INVALID_CONFIG: return "no such tile-table entry";
    case GEMM_ERR_SCRATCH_TOO_SMALL:
        return "split-K partial sums exceed the 32 MiB scratch of gemm_run_noalloc";
    default: return "unknown status";
    }
}

int gemm_num_configs(void) { return kNumConfigs; }

const char *gemm_config_name(int config_id) {
    if (config_id < 0 || config_id >= kNumConfigs) return nullptr;
    return kTable[config_id].name;
}

int gemm_select_config(int64_t M, int64_t N, int64_t K, int layoutA, int layoutB, int in_dtype,
                       int acc_dtype, int out_dtype) {
    // validate everything that does not involve pointers or leading dims
    const int st = validate(M, N, K, nullptr, 1 + (layoutA == GEMM_ROW_MAJOR ? K : M), layoutA,
                            nullptr, 1 + (layoutB == GEMM_ROW_MAJOR ? N : K), layoutB, nullptr,
                            1 + N, nullptr, 1 + N, in_dtype, acc_dtype, out_dtype, nullptr, 0);
    if (st != GEMM_OK && st != GEMM_ERR_NULL_PTR) return st;
    return refine_large(select_config(M, N, K, input_class(in_dtype), topology().cus), true,
                        layoutA, layoutB, K);
}

}  // extern "C"
