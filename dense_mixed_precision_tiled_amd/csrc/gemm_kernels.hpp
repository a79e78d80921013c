// Tiled MFMA kernels for D = A x B + C on gfx950 (MI355X, CDNA4).
//
// One workgroup computes one BM x BN tile of D (optionally one K-slice of it,
// for split-K).  Per K-tile of depth BK:
//   global -> registers : 16-byte loads, adjacent lanes on adjacent addresses;
//                         operands whose rows are contiguous along M/N are
//                         transposed in registers on the way, so LDS always
//                         holds both operands K-contiguous;
//   registers -> LDS    : XOR-swizzled 16-byte chunks (conflict-free for
//                         both the writes and the MFMA operand reads);
//   LDS -> registers    : one 16-byte read per lane per MFMA operand;
//   MFMA                : v_mfma_f32_32x32x16_{f16,bf16} or
//                         v_mfma_f32_16x16x32_{f16,bf16}, fp32 accumulators
//                         held in registers, TM x TN tiles per wave.
// Two LDS stages: the loads of K-tile t+1 are in flight while tile t is
// multiplied, with one barrier per K-tile.  Edge tiles (ragged M, N, K, or
// unaligned operands) take a checked path that zero-fills what lies outside
// the matrices; interior tiles take the unchecked vector path.
//
// Sources for the method (page title, section):
//  - hierarchical tiling, C tile per block, K sliced by BLOCK_K, fp32
//    accumulators in registers: "矩阵乘法优化可视化学习文档", sections 4
//    "Tiling" and 6 "常用优化方法总表";
//  - shared-memory staging with barriers after the store and before reuse:
//    "CUDA算子优化(5)：WMMA矩阵乘法", section "WMMA共享内存";
//  - zero-filled edges, bank-conflict padding, double buffering:
//    "深入CUDA Tensor Core与WMMA…", sections 5.2, 5.3 and 5.4;
//  - vectorised 128-bit global access, register tiling: same page,
//    section 5.5, and "矩阵乘法优化可视化学习文档" section 6;
//  - epilogue (C add, convert, satf) fused before the store:
//    "CUDA算子优化(5)：WMMA矩阵乘法", section "WMMA API解释" item (5), and
//    "矩阵乘法优化可视化学习文档" section 6 (Epilogue fusion row).
// The pages' WMMA / mma.sync designs target NVIDIA warps; this kernel keeps
// their ideas and is laid out for 64-lane waves, MFMA and gfx950's LDS.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "gemm_address.hpp"

namespace libgemm {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef int32_t i32x2 __attribute__((ext_vector_type(2)));
typedef int32_t i32x16 __attribute__((ext_vector_type(16)));

// dtype codes of the C ABI (C, D and out_dtype)
enum { DT_F32 = 0, DT_F16 = 1, DT_BF16 = 2, DT_I8 = 3, DT_I32 = 4 };
// input (A, B) element types of the kernels: fp16, bf16, int8, OCP fp8 E4M3, E5M2
enum { IT_F16 = 0, IT_BF16 = 1, IT_I8 = 2, IT_FP8 = 3, IT_BF8 = 4 };
typedef int32_t i32x8 __attribute__((ext_vector_type(8)));

// Compile-time loop: f(integral_constant<int, I>) for I in [B, E).  Keeps
// every accumulator index a constant so the accumulators stay in registers.
template <int B, int E>
struct Unroll {
    template <class F>
    __device__ __forceinline__ static void run(F &&f) {
        f(std::integral_constant<int, B>{});
        Unroll<B + 1, E>::run(f);
    }
};
template <int E>
struct Unroll<E, E> {
    template <class F>
    __device__ __forceinline__ static void run(F &&) {}
};

// Everything a launch needs; passed by value as the kernel argument.
struct Params {
    const uint16_t *A;
    const uint16_t *B;
    const void *C;   // out_dtype elements, row-major, or nullptr
    void *D;         // out_dtype elements, row-major
    float *ws;       // split-K partial sums [splits][M][N], or nullptr
    int64_t lda, ldb, ldc, ldd;
    int M, N, K;
    int out_dtype;
    int satf;
    int vec_ok;      // A, B 16-byte aligned with lda, ldb multiples of 8
    int cd_vec;      // C, D rows allow 4-element vector access (aligned base, ld % 4 == 0)
    uint32_t a_bytes, b_bytes;  // vector path: A, B extents rounded up to 16 bytes
    int tiles_m, tiles_n;
    int group_m;     // tile-rows per raster group (see raster_tile)
    int skew;        // raster groups start at staggered columns (see raster_tile)
    int xcds;        // XCDs the device hands workgroups to (round-robin)
    int splits;      // K slices (blockIdx.z); 1 = no split
    int k_per_split; // multiple of BK
    // extended epilogue: v = act(alpha * sum + beta * C + bias).  epi == 0 is
    // the plain v = sum + C (alpha = beta = 1, no bias, no activation).
    int epi;
    float alpha, beta;
    const float *bias;  // fp32, indexed by column (or by row with bias_rows), or nullptr
    int bias_rows;
    int act;            // ACT_*
    int c_col;          // C column-major: C(i,j) = C[j*ldc + i]
};

enum { ACT_NONE = 0, ACT_RELU = 1, ACT_GELU = 2 };

// Block-tile configuration.  MF = 32 selects the 32x32 MFMA (32x32x16 for
// 16-bit inputs, 32x32x32 for int8, 32x32x64 for fp8), 16 the 16x16 one
// (16x16x32, 16x16x64, 16x16x128).  Waves form a WAVES_M x WAVES_N grid over
// the block tile.  ES is the input element size in bytes; BK counts
// elements, so an LDS row holds BK*ES bytes.  FC is the number of 16-byte
// chunks of each operand one lane holds per MFMA: 1 for the 16-bit and int8
// MFMAs, 2 for the fp8 ones.  In bytes, the tiles of every type share one
// LDS layout.
template <int BM_, int BN_, int BK_, int WAVES_M_, int WAVES_N_, int MF_, int ES_ = 2, int FC_ = 1>
struct TileCfg {
    static constexpr int BM = BM_, BN = BN_, BK = BK_;
    static constexpr int WAVES_M = WAVES_M_, WAVES_N = WAVES_N_;
    static constexpr int THREADS = 64 * WAVES_M * WAVES_N;
    static constexpr int MF = MF_;
    static constexpr int ES = ES_;
    static constexpr int FC = FC_;
    static constexpr int KSTEP = FC * ((MF == 32) ? 32 : 64) / ES;  // k consumed by one MFMA
    static constexpr int WTM = BM / WAVES_M, WTN = BN / WAVES_N;
    static constexpr int TM = WTM / MF, TN = WTN / MF;
    static constexpr int CH = BK * ES / 16;  // 16-byte chunks per LDS row
    static_assert(MF == 32 || MF == 16, "MFMA shape");
    static_assert(ES == 1 || ES == 2, "element size");
    static_assert((BK * ES) % 128 == 0, "the LDS swizzle assumes rows of >= 128 bytes");
    static_assert(WTM % MF == 0 && WTN % MF == 0, "wave tile");
    static_assert(BM % 8 == 0 && BN % 8 == 0, "row groups of 8");
};

// ---------------------------------------------------------------- LDS layout
// Row r of an operand tile holds BK k-values (CH 16-byte chunks).  Chunk c is
// stored at position c ^ swz(r).  Eight consecutive rows read at one chunk,
// and eight rows 8 apart written at one chunk, land in eight different
// 16-byte bank groups.
__device__ __forceinline__ int swz(int r) { return swz_kc(r); }

// ------------------------------------------------------------ small helpers
__device__ __forceinline__ uint32_t lo16(uint32_t x) { return x & 0xffffu; }
__device__ __forceinline__ uint32_t hi16(uint32_t x) { return x >> 16; }

// Element e (0..7) of a 16-byte vector of 16-bit values.
__device__ __forceinline__ uint32_t half_of(const u32x4 &v, int e) {
    uint32_t d = v[e >> 1];
    return (e & 1) ? hi16(d) : lo16(d);
}

// ---------------------------------------------------------------- loaders
// Operand X with "rows" r (M for A, N for B) and depth k.
//  K-contiguous storage: X(r,k) = X[r*ld + k]   (row-major A, col-major B)
//  R-contiguous storage: X(r,k) = X[k*ld + r]   (col-major A, row-major B)
// Each loader fetches one ROWS x BK tile into registers and writes it to LDS
// K-contiguous (store).
//
// Vector path (16-byte aligned operands, extent < 4 GiB): 16-byte buffer
// loads through a descriptor whose range is the operand's extent rounded up
// to 16 bytes.  Rows beyond R are clamped to the last valid row (8-row
// chunk): they only feed outputs that are never stored.  Per-lane offsets
// are fixed for the K loop and the K position goes in the scalar offset,
// except in RAGGED kernels (K not a multiple of BK): there the k position is
// part of the per-lane offset and clamped to the chunk holding kend-1, and
// the loaded values for k >= kend are masked to zero.  So every chunk read
// holds an element of the matrix (gemm_address.hpp), whatever the range
// check does with the scalar offset.
// Threads beyond a small tile's chunk count duplicate a chunk (same value to
// the same LDS address), which keeps the code free of branches.
//
// Checked path (unaligned operands): element-wise loads with zero fill.

// Keep the first n (0..8) 16-bit elements of a 16-byte chunk, zero the rest.
__device__ __forceinline__ u32x4 keep_first(u32x4 v, int n) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const uint32_t m = (2 * q + 1 < n) ? 0xffffffffu : (2 * q < n ? 0x0000ffffu : 0u);
        v[q] &= m;
    }
    return v;
}

// Keep the first n (0..16) bytes of a 16-byte chunk, zero the rest.
__device__ __forceinline__ u32x4 keep_first_bytes(u32x4 v, int n) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int b = n - 4 * q;  // bytes of dword q to keep
        const uint32_t m = b >= 4 ? 0xffffffffu : (b <= 0 ? 0u : ((1u << (8 * b)) - 1u));
        v[q] &= m;
    }
    return v;
}

__device__ __forceinline__ u32x4 buf_load16(__amdgpu_buffer_rsrc_t rsrc, uint32_t voff,
                                            uint32_t soff) {
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rsrc, (int)voff,
                                                                            (int)soff, 0));
}
__device__ __forceinline__ uint32_t buf_load4(__amdgpu_buffer_rsrc_t rsrc, uint32_t voff,
                                             uint32_t soff) {
    return __builtin_amdgcn_raw_buffer_load_b32(rsrc, (int)voff, (int)soff, 0);
}

template <int ROWS, int BK, int THREADS, int ES = 2>
struct LoaderKC {
    static constexpr int CH = BK * ES / 16;
    static constexpr int EPC = 16 / ES;  // elements per 16-byte chunk
    static constexpr int TOTAL = ROWS * CH;  // 16-byte chunks in the tile
    static constexpr bool PARTIAL = TOTAL < THREADS;
    static constexpr int PER = PARTIAL ? 1 : TOTAL / THREADS;
    static constexpr int NLOAD = PER, NSTORE = PER;
    static constexpr int SPB = 1, LPB = 1;  // stores and loads per block (a chunk)
    static_assert(PARTIAL || TOTAL % THREADS == 0, "tile/threads");
    static_assert(PARTIAL || THREADS % CH == 0, "threads/chunks");
    u32x4 v[PER];
    uint32_t voff[PER];  // byte offset of each chunk at k0 = 0 (row clamped)
    int kc;              // this thread's k offset inside the K-tile

    __device__ __forceinline__ static int chunk(int i, int tid) {
        return PARTIAL ? tid % TOTAL : i * THREADS + tid;
    }

    __device__ __forceinline__ void init(int tid, int64_t ld, int r0, int R) {
        kc = (chunk(0, tid) % CH) * EPC;
#pragma unroll
        for (int i = 0; i < PER; ++i)
            voff[i] = (uint32_t)kc_chunk_offset(r0 + chunk(i, tid) / CH, kc, R, 1, ld, ES, false);
    }

    // CLAMPK (kernels whose last K-tile is ragged): the k position goes into
    // the per-lane offset, clamped to the chunk holding kend-1; otherwise it
    // rides in the scalar offset (every k of every K-tile is < kend).
    template <bool CLAMPK>
    __device__ __forceinline__ u32x4 load_at(__amdgpu_buffer_rsrc_t rsrc, int i, int k0,
                                             int kend) const {
        if constexpr (CLAMPK)
            return buf_load16(rsrc, voff[i] - (uint32_t)(kc * ES) +
                                        (uint32_t)kc_k_offset(k0 + kc, kend, ES), 0u);
        else
            return buf_load16(rsrc, voff[i], (uint32_t)k0 * (uint32_t)ES);
    }

    template <bool CLAMPK>
    __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t rsrc, int k0, int64_t, int kend) {
#pragma unroll
        for (int i = 0; i < PER; ++i) v[i] = load_at<CLAMPK>(rsrc, i, k0, kend);
    }

    // the idx-th global load / LDS store of load() / store(), one instruction
    template <int idx, bool CLAMPK>
    __device__ __forceinline__ void load_one(__amdgpu_buffer_rsrc_t rsrc, int k0, int64_t,
                                             int kend) {
        v[idx] = load_at<CLAMPK>(rsrc, idx, k0, kend);
    }
    template <int idx>
    __device__ __forceinline__ void store_one(u32x4 *lds, int tid) const {
        const int q = chunk(idx, tid);
        const int r = q / CH, c = q % CH;
        lds[r * CH + (c ^ swz(r))] = v[idx];
    }

    __device__ __forceinline__ void mask(int k0, int kend) {
        const int n = min(max(kend - (k0 + kc), 0), EPC);
#pragma unroll
        for (int i = 0; i < PER; ++i) v[i] = ES == 2 ? keep_first(v[i], n) : keep_first_bytes(v[i], n);
    }

    // Element-wise loads with zero fill.  RCADDR: the operand is stored
    // R-contiguous (X(r,k) = X[k*ld + r]); the chunks are still K-contiguous.
    template <bool RCADDR>
    __device__ __forceinline__ void load_checked(const uint16_t *X, int64_t ld, int r0, int k0,
                                                 int R, int Kend, int tid) {
        const uint8_t *X8 = reinterpret_cast<const uint8_t *>(X);
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int q = chunk(i, tid);
            const int r = q / CH, c = q % CH;
            const int gr = r0 + r, gk = k0 + c * EPC;
            uint32_t h[EPC];
#pragma unroll
            for (int e = 0; e < EPC; ++e) {
                const int64_t off = RCADDR ? (int64_t)(gk + e) * ld + gr : (int64_t)gr * ld + gk + e;
                const bool in = gr < R && gk + e < Kend;
                h[e] = in ? (ES == 2 ? (uint32_t)X[off] : (uint32_t)X8[off]) : 0u;
            }
            if constexpr (ES == 2) {
                v[i] = u32x4{h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16),
                             h[6] | (h[7] << 16)};
            } else {
#pragma unroll
                for (int d = 0; d < 4; ++d)
                    v[i][d] = h[4 * d] | (h[4 * d + 1] << 8) | (h[4 * d + 2] << 16) |
                              (h[4 * d + 3] << 24);
            }
        }
    }

    __device__ __forceinline__ void store(u32x4 *lds, int tid) const {
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int q = chunk(i, tid);
            const int r = q / CH, c = q % CH;
            lds[r * CH + (c ^ swz(r))] = v[i];
        }
    }
};

template <int ROWS, int BK, int THREADS>
struct LoaderRC {
    static constexpr int RCH = ROWS / 8;        // 8-row chunks along one k
    static constexpr int TOTAL = RCH * BK;      // 16-byte chunks in the tile
    static constexpr bool PARTIAL = TOTAL < THREADS;
    static constexpr int PERT = PARTIAL ? 1 : TOTAL / THREADS;
    static constexpr int KB = PERT < 8 ? PERT : 8;   // k-depth of one block
    static constexpr int NBLK = PERT / KB;           // blocks per thread
    static constexpr int NBLOCKS = TOTAL / KB;       // blocks in the tile
    static constexpr int NLOAD = NBLK * KB, NSTORE = NBLK * 8;
    static constexpr int SPB = 8, LPB = KB;  // stores and loads per block
    static_assert(PARTIAL || TOTAL % THREADS == 0, "tile/threads");
    static_assert(KB == 1 || KB == 2 || KB == 4 || KB == 8, "k-depth");
    static_assert(PERT % KB == 0, "blocks");
    static_assert(BK % KB == 0, "k groups");
    static_assert(PARTIAL || THREADS % RCH == 0, "threads/row chunks");
    // Block b -> (8-row chunk rb, k-group kg).  PAIRS: two adjacent lanes
    // take the same rb at two adjacent k-groups, and adjacent pairs adjacent
    // 16 bytes of a k-row (the global loads stay coalesced).  Then one
    // transposing store instruction of 32 lanes writes both 8-byte halves of
    // the LDS chunks it touches, twice the banks of the plain mapping
    // (rb = b % RCH), whose 32 lanes hit a quarter of the banks 4 deep.
    static constexpr bool PAIRS =
        (NBLOCKS % (2 * RCH) == 0) && (PARTIAL || THREADS % (2 * RCH) == 0);
    u32x4 v[NBLK][KB];  // v[j][kk]: 8 consecutive r at k = kg_j*KB + kk
    uint32_t voff;      // byte offset of this thread's 8-row chunk at k = 0
    int kg[NBLK];       // k-group of each block

    __device__ __forceinline__ static int block(int j, int tid) {
        return PARTIAL ? tid % NBLOCKS : j * THREADS + tid;
    }
    __device__ __forceinline__ static int rb_of(int b) { return PAIRS ? (b >> 1) % RCH : b % RCH; }
    __device__ __forceinline__ static int kg_of(int b) {
        return PAIRS ? (b & 1) + 2 * (b / (2 * RCH)) : b / RCH;
    }

    __device__ __forceinline__ void init(int tid, int64_t /*ld: per load*/, int r0, int R) {
        const int rb = rb_of(block(0, tid));   // the same for every j
        voff = (uint32_t)rc_chunk_offset(r0 + rb * 8, 0, R, 1, 0, false);
#pragma unroll
        for (int j = 0; j < NBLK; ++j) kg[j] = kg_of(block(j, tid));
    }

    // CLAMPK: the row k goes into the per-lane offset, clamped to kend-1;
    // otherwise the K-tile's start rides in the scalar offset
    template <bool CLAMPK>
    __device__ __forceinline__ u32x4 load_at(__amdgpu_buffer_rsrc_t rsrc, int j, int kk, int k0,
                                             int64_t ld, int kend) const {
        const uint32_t ldb = (uint32_t)ld * 2u;
        if constexpr (CLAMPK)
            return buf_load16(rsrc, voff + (uint32_t)imin(k0 + kg[j] * KB + kk, kend - 1) * ldb, 0u);
        else
            return buf_load16(rsrc, voff + (uint32_t)(kg[j] * KB + kk) * ldb, (uint32_t)k0 * ldb);
    }

    template <bool CLAMPK>
    __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t rsrc, int k0, int64_t ld, int kend) {
#pragma unroll
        for (int j = 0; j < NBLK; ++j)
#pragma unroll
            for (int kk = 0; kk < KB; ++kk) v[j][kk] = load_at<CLAMPK>(rsrc, j, kk, k0, ld, kend);
    }

    template <int idx, bool CLAMPK>
    __device__ __forceinline__ void load_one(__amdgpu_buffer_rsrc_t rsrc, int k0, int64_t ld,
                                             int kend) {
        constexpr int j = idx / KB, kk = idx % KB;
        v[j][kk] = load_at<CLAMPK>(rsrc, j, kk, k0, ld, kend);
    }

    __device__ __forceinline__ void mask(int k0, int kend) {
#pragma unroll
        for (int j = 0; j < NBLK; ++j)
#pragma unroll
            for (int kk = 0; kk < KB; ++kk)
                if (k0 + kg[j] * KB + kk >= kend) v[j][kk] = u32x4{0u, 0u, 0u, 0u};
    }

    template <bool RCADDR>  // always R-contiguous here
    __device__ __forceinline__ void load_checked(const uint16_t *X, int64_t ld, int r0, int k0,
                                                 int R, int Kend, int tid) {
#pragma unroll
        for (int j = 0; j < NBLK; ++j) {
            const int b = block(j, tid);
            const int rb = rb_of(b), kgb = kg_of(b);
            const int gr = r0 + rb * 8;
#pragma unroll
            for (int kk = 0; kk < KB; ++kk) {
                const int gk = k0 + kgb * KB + kk;
                const uint16_t *src = X + (int64_t)gk * ld + gr;
                uint32_t h[8];
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    h[e] = (gk < Kend && gr + e < R) ? (uint32_t)src[e] : 0u;
                v[j][kk] = u32x4{h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16),
                                 h[6] | (h[7] << 16)};
            }
        }
    }

    // the idx-th LDS store of store(): block idx / 8, column idx % 8
    template <int idx>
    __device__ __forceinline__ void store_one(u32x4 *lds, int tid) const {
        store_col(lds, tid, idx / 8, idx % 8);
    }

    // {element e of a, element e of b} packed into one dword (low half from
    // a): one v_perm_b32 (byte select from the pair {b, a}, a supplying bytes
    // 0-3)
    __device__ __forceinline__ static uint32_t pair_of(const u32x4 &a, const u32x4 &b, int e) {
        return __builtin_amdgcn_perm(b[e >> 1], a[e >> 1], (e & 1) ? 0x07060302u : 0x05040100u);
    }

    // Transpose block j in registers: LDS row rb*8 + e receives the KB
    // k-values of column e, at k offset kg*KB.
    __device__ __forceinline__ void store_col(u32x4 *lds, int tid, int j, int e) const {
        constexpr int CH = BK / 8;
        const int b = block(j, tid);
        const int rb = rb_of(b), kgb = kg_of(b);
        const int kofs = kgb * KB;
        const int c = kofs / 8, sub = kofs % 8;  // chunk and element offset
        const int r = rb * 8 + e;
        u32x4 *dst = lds + r * CH + (c ^ swz(r));
        if constexpr (KB == 8) {
            u32x4 w;
#pragma unroll
            for (int q = 0; q < 4; ++q) w[q] = pair_of(v[j][2 * q], v[j][2 * q + 1], e);
            *dst = w;
        } else if constexpr (KB == 4) {
            u32x2 w;
            w[0] = pair_of(v[j][0], v[j][1], e);
            w[1] = pair_of(v[j][2], v[j][3], e);
            reinterpret_cast<u32x2 *>(dst)[sub / 4] = w;
        } else if constexpr (KB == 2) {
            reinterpret_cast<uint32_t *>(dst)[sub / 2] = pair_of(v[j][0], v[j][1], e);
        } else {
            reinterpret_cast<uint16_t *>(dst)[sub] = (uint16_t)half_of(v[j][0], e);
        }
    }

    __device__ __forceinline__ void store(u32x4 *lds, int tid) const {
#pragma unroll
        for (int j = 0; j < NBLK; ++j)
#pragma unroll
            for (int e = 0; e < 8; ++e) store_col(lds, tid, j, e);
    }
};

// R-contiguous 8-bit operand (row-major B or column-major A of int8 / fp8):
// blocks of 4 consecutive rows r x 16 k-rows, one dword load per k-row (the
// lanes of a wave cover consecutive 4-row groups, so one load instruction
// reads a contiguous stretch of a k-row), transposed in registers into the
// 16-byte K-contiguous chunks of the 4 rows (rc8_gather), which go to LDS
// like the K-contiguous loader's.  A tile with fewer blocks than threads has
// threads repeat blocks (identical stores).
template <int ROWS, int BK, int THREADS>
struct LoaderRC8 {
    static constexpr int CH = BK / 16;             // 16-byte chunks per LDS row
    static constexpr int RG = ROWS / 4;             // 4-row groups
    static constexpr int TOTAL = RG * (BK / 16);    // blocks in the tile
    static constexpr bool PARTIAL = TOTAL < THREADS;
    static constexpr int NBLK = PARTIAL ? 1 : TOTAL / THREADS;
    static constexpr int NLOAD = NBLK * 16, NSTORE = NBLK * 4;
    static constexpr int SPB = 4, LPB = 16;         // stores and loads per block
    static_assert(ROWS % 4 == 0 && BK % 16 == 0, "4-row groups, 16 k-rows per block");
    static_assert(PARTIAL || TOTAL % THREADS == 0, "tile/threads");
    static_assert(PARTIAL || THREADS % RG == 0, "threads/row groups");
    uint32_t v[NBLK][16];  // v[j][kk]: rows 4rg..4rg+3 at k = 16*kg_j + kk
    uint32_t voff;         // byte offset of this thread's row group at k = 0
    int rg;                // the row group (the same for every j)
    int kg[NBLK];          // k-group of each block

    __device__ __forceinline__ static int block(int j, int tid) {
        return PARTIAL ? tid % TOTAL : j * THREADS + tid;
    }

    __device__ __forceinline__ void init(int tid, int64_t ld, int r0, int R) {
        rg = block(0, tid) % RG;
        voff = (uint32_t)rc8_dword_offset(r0 + rg * 4, 0, R, 1, ld, false);
#pragma unroll
        for (int j = 0; j < NBLK; ++j) kg[j] = block(j, tid) / RG;
    }

    // CLAMPK: the k-row goes into the per-lane offset, clamped to kend-1;
    // otherwise the K-tile's start rides in the scalar offset
    template <bool CLAMPK>
    __device__ __forceinline__ uint32_t load_at(__amdgpu_buffer_rsrc_t rsrc, int j, int kk, int k0,
                                                int64_t ld, int kend) const {
        const uint32_t l = (uint32_t)ld;
        if constexpr (CLAMPK)
            return buf_load4(rsrc, voff + (uint32_t)imin(k0 + kg[j] * 16 + kk, kend - 1) * l, 0u);
        else
            return buf_load4(rsrc, voff + (uint32_t)(kg[j] * 16 + kk) * l, (uint32_t)k0 * l);
    }

    template <bool CLAMPK>
    __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t rsrc, int k0, int64_t ld, int kend) {
#pragma unroll
        for (int j = 0; j < NBLK; ++j)
#pragma unroll
            for (int kk = 0; kk < 16; ++kk) v[j][kk] = load_at<CLAMPK>(rsrc, j, kk, k0, ld, kend);
    }

    template <int idx, bool CLAMPK>
    __device__ __forceinline__ void load_one(__amdgpu_buffer_rsrc_t rsrc, int k0, int64_t ld,
                                             int kend) {
        v[idx / 16][idx % 16] = load_at<CLAMPK>(rsrc, idx / 16, idx % 16, k0, ld, kend);
    }

    __device__ __forceinline__ void mask(int k0, int kend) {
#pragma unroll
        for (int j = 0; j < NBLK; ++j)
#pragma unroll
            for (int kk = 0; kk < 16; ++kk)
                if (k0 + kg[j] * 16 + kk >= kend) v[j][kk] = 0u;
    }

    // the idx-th LDS store: block idx / 4, row 4rg + idx % 4 (the thread's
    // blocks are fixed at init; tid keeps the loaders' common signature)
    template <int idx>
    __device__ __forceinline__ void store_one(u32x4 *lds, int /*tid*/) const {
        constexpr int j = idx / 4, e = idx % 4;
        u32x4 w;
#pragma unroll
        for (int d = 0; d < 4; ++d)
            w[d] = rc8_gather(v[j][4 * d], v[j][4 * d + 1], v[j][4 * d + 2], v[j][4 * d + 3], e);
        const int r = rg * 4 + e;
        lds[r * CH + (kg[j] ^ swz(r))] = w;
    }

    __device__ __forceinline__ void store(u32x4 *lds, int tid) const {
        Unroll<0, NSTORE>::run([&](auto w) { store_one<decltype(w)::value>(lds, tid); });
    }
};

// ------------------------------------------------------------------- MFMA
// int8: the accumulators hold int32 bit patterns in the same float vectors
// (only moved, never used as floats until the epilogue reinterprets them).
template <int IT>
__device__ __forceinline__ f32x16 mfma32_1(const u32x4 &a, const u32x4 &b, const f32x16 &c) {
    if constexpr (IT == IT_BF16)
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
    else if constexpr (IT == IT_F16)
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                      __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
    else
        return __builtin_bit_cast(
            f32x16, __builtin_amdgcn_mfma_i32_32x32x32_i8(__builtin_bit_cast(i32x4, a),
                                                           __builtin_bit_cast(i32x4, b),
                                                           __builtin_bit_cast(i32x16, c), 0, 0, 0));
}

template <int IT>
__device__ __forceinline__ f32x4 mfma16_1(const u32x4 &a, const u32x4 &b, const f32x4 &c) {
    if constexpr (IT == IT_BF16)
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
    else if constexpr (IT == IT_F16)
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                      __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
    else
        return __builtin_bit_cast(
            f32x4, __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_bit_cast(i32x4, a),
                                                          __builtin_bit_cast(i32x4, b),
                                                          __builtin_bit_cast(i32x4, c), 0, 0, 0));
}

// fp8 operands: two 16-byte chunks per lane; scale exponents 127 (= 2^0).
__device__ __forceinline__ i32x8 cat8(const u32x4 &lo, const u32x4 &hi) {
    return i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                 (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
}

template <int IT, int FC>
__device__ __forceinline__ f32x16 mfma32(const u32x4 (&af)[FC], const u32x4 (&bf)[FC],
                                         const f32x16 &c) {
    if constexpr (IT == IT_FP8 || IT == IT_BF8) {
        constexpr int fmt = IT == IT_FP8 ? 0 : 1;
        return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
            cat8(af[0], af[FC - 1]), cat8(bf[0], bf[FC - 1]), c, fmt, fmt, 0, 127, 0, 127);
    } else {
        return mfma32_1<IT>(af[0], bf[0], c);
    }
}

template <int IT, int FC>
__device__ __forceinline__ f32x4 mfma16(const u32x4 (&af)[FC], const u32x4 (&bf)[FC],
                                        const f32x4 &c) {
    if constexpr (IT == IT_FP8 || IT == IT_BF8) {
        constexpr int fmt = IT == IT_FP8 ? 0 : 1;
        return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
            cat8(af[0], af[FC - 1]), cat8(bf[0], bf[FC - 1]), c, fmt, fmt, 0, 127, 0, 127);
    } else {
        return mfma16_1<IT>(af[0], bf[0], c);
    }
}

template <int MF> struct AccT;
template <> struct AccT<32> { typedef f32x16 type; static constexpr int N = 16; };
template <> struct AccT<16> { typedef f32x4 type; static constexpr int N = 4; };

// Position of accumulator register r of `lane` inside an MF x MF tile of D.
// The MFMA output layout (column lane % MF; rows 8*(r/4) + 4*(lane/32) + r%4
// for 32x32, 4*(lane/16) + r for 16x16) describes the transposed tile here,
// because the operands are passed B first.  So lane holds D row lane % MF,
// and registers 4g..4g+3 hold four consecutive D columns starting at
// acc_col(lane, g).
template <int MF>
__device__ __forceinline__ int acc_row(int lane) { return lane & (MF - 1); }
template <int MF>
__device__ __forceinline__ int acc_col(int lane, int g) {
    if constexpr (MF == 32)
        return 8 * g + 4 * (lane >> 5);
    else
        return 4 * (lane >> 4);
}

// ---------------------------------------------------------------- epilogue
__device__ __forceinline__ float load_c(const Params &p, int64_t i, int64_t j) {
    const int64_t off = p.c_col ? j * p.ldc + i : i * p.ldc + j;
    if (p.out_dtype == DT_F32) return reinterpret_cast<const float *>(p.C)[off];
    const uint16_t h = reinterpret_cast<const uint16_t *>(p.C)[off];
    if (p.out_dtype == DT_F16) return (float)__builtin_bit_cast(_Float16, h);
    return __uint_as_float((uint32_t)h << 16);
}

// fp32 -> bf16, round to nearest even (NaN stays a quiet NaN).
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float x) {
    uint32_t u = __float_as_uint(x);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// GELU(x) = x * Phi(x), Phi(x) = 1 - erfc(x / sqrt 2) / 2 for x >= 0 and
// erfc(|x| / sqrt 2) / 2 for x < 0, with erfc from Abramowitz & Stegun,
// "Handbook of Mathematical Functions", formula 7.1.26:
//   erfc(z) ~ t (a1 + t (a2 + t (a3 + t (a4 + t a5)))) exp(-z^2),
//   t = 1 / (1 + p z),   |error| <= 1.5e-7 for z >= 0.
// Forming Phi from erfc avoids the cancellation of 1 + erf for x << 0, so
// the absolute error of GELU stays below about 1e-7 * |x|.  Branch-free but
// for the select on the sign; +-Inf take GELU's limits, NaN stays NaN.
__device__ __forceinline__ float gelu_f32(float x) {
    if (__builtin_isinf(x)) return x > 0.0f ? x : 0.0f;
    const float z = __builtin_fabsf(x) * 0.70710678118654752f;
    const float t = __builtin_amdgcn_rcpf(1.0f + 0.3275911f * z);
    const float poly =
        t * (0.254829592f +
             t * (-0.284496736f + t * (1.421413741f + t * (-1.453152027f + t * 1.061405429f))));
    const float q = poly * __expf(-z * z);  // erfc(z)
    const float phi = x >= 0.0f ? 1.0f - 0.5f * q : 0.5f * q;
    return x * phi;
}

// ReLU keeps NaN and maps -0 to +0.
__device__ __forceinline__ float activate(float x, int act) {
    if (act == ACT_RELU) return (x > 0.0f || x != x) ? x : 0.0f;
    if (act == ACT_GELU) return gelu_f32(x);
    return x;
}

// The epilogue of one element before the rounding: sum (+ C), or with the
// extended epilogue act(alpha * sum + beta * C + bias).
__device__ __forceinline__ float epilogue_value(const Params &p, int64_t i, int64_t j, float v) {
    if (!p.epi) return p.C ? v + load_c(p, i, j) : v;
    v = p.alpha * v;
    if (p.C) v += p.beta * load_c(p, i, j);
    if (p.bias) v += p.bias[p.bias_rows ? i : j];
    return activate(v, p.act);
}

// The epilogue value of D(i,j), rounded once to the output dtype OUT, then
// satf, stored at D(i,j).  OUT is a template argument so the hot epilogue has
// no dtype branch.
template <int OUT>
__device__ __forceinline__ void finish_store_t(const Params &p, int64_t i, int64_t j, float v) {
    v = epilogue_value(p, i, j, v);
    const int64_t off = i * p.ldd + j;
    if constexpr (OUT == DT_F32) {
        if (p.satf) {
            if (__builtin_isnan(v)) v = 0.0f;
            else if (__builtin_isinf(v)) v = v > 0 ? 3.402823466e38f : -3.402823466e38f;
        }
        reinterpret_cast<float *>(p.D)[off] = v;
    } else {
        constexpr uint16_t expo = (OUT == DT_F16) ? 0x7c00u : 0x7f80u;
        constexpr uint16_t mx = (OUT == DT_F16) ? 0x7bffu : 0x7f7fu;
        uint16_t h;
        if constexpr (OUT == DT_F16)
            h = __builtin_bit_cast(uint16_t, (_Float16)v);
        else
            h = f32_to_bf16_rne(v);
        if (p.satf && (h & expo) == expo) {
            if (h & (uint16_t)(~expo & 0x7fffu)) h = 0;          // NaN -> +0
            else h = (uint16_t)((h & 0x8000u) | mx);           // +-Inf -> +-MAX_NORM
        }
        reinterpret_cast<uint16_t *>(p.D)[off] = h;
    }
}

__device__ __forceinline__ void finish_store(const Params &p, int64_t i, int64_t j, float v) {
    if (p.out_dtype == DT_F32) finish_store_t<DT_F32>(p, i, j, v);
    else if (p.out_dtype == DT_F16) finish_store_t<DT_F16>(p, i, j, v);
    else finish_store_t<DT_BF16>(p, i, j, v);
}

// int64 -> int32: modulo 2^32, or with satf clamped to the int32 range.
__device__ __forceinline__ int32_t to_int32(int64_t t, int satf) {
    if (satf) return (int32_t)(t > INT32_MAX ? INT32_MAX : (t < INT32_MIN ? INT32_MIN : t));
    return (int32_t)(uint32_t)(uint64_t)t;
}

// satf on a rounded fp32 value: +-Inf -> +-MAX_NORM, NaN -> +0.
__device__ __forceinline__ float satf_f32(float x) {
    if (__builtin_isnan(x)) return 0.0f;
    if (__builtin_isinf(x)) return x > 0 ? 3.402823466e38f : -3.402823466e38f;
    return x;
}

// fp32 -> 16-bit output pattern (RNE), then satf when asked.
template <int OUT>
__device__ __forceinline__ uint32_t to_out16(float x, bool satf) {
    constexpr uint32_t expo = (OUT == DT_F16) ? 0x7c00u : 0x7f80u;
    constexpr uint32_t mx = (OUT == DT_F16) ? 0x7bffu : 0x7f7fu;
    uint32_t h = (OUT == DT_F16) ? (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)x)
                                 : (uint32_t)f32_to_bf16_rne(x);
    if (satf && (h & expo) == expo)
        h = (h & (~expo & 0x7fffu)) ? 0u : ((h & 0x8000u) | mx);
    return h;
}

template <int OUT>
__device__ __forceinline__ float from_out16(uint32_t h) {
    return (OUT == DT_F16) ? (float)__builtin_bit_cast(_Float16, (uint16_t)h)
                           : __uint_as_float(h << 16);
}

// Four consecutive outputs D(i, j..j+3) from fp32 sums v.  OUT < 0: split-K
// slice, store the raw sums to the workspace.  Otherwise the epilogue is
// applied (EPI: the extended act(alpha*v + beta*C + bias), else v + C), the
// result rounded once to OUT, satf applied and the group stored.  FULL: the
// group lies inside M x N and C/D/bias allow 4-element vector access, so no
// checks; else each element is checked and stored alone.
// C(i, j..j+3) of a group inside M x N with vector-friendly row-major C (float
// outputs only), as raw bits (fp32: 4 words; 16-bit: 2 words of two values
// each), so that a batch of loads holds half the registers until its values
// are used; c_from_raw converts them to fp32.
template <int OUT>
__device__ __forceinline__ auto load_c_raw(const Params &p, int i, int j) {
    if constexpr (OUT == DT_F32) {
        return *reinterpret_cast<const u32x4 *>(reinterpret_cast<const float *>(p.C) +
                                                (int64_t)i * p.ldc + j);
    } else {
        return *reinterpret_cast<const u32x2 *>(reinterpret_cast<const uint16_t *>(p.C) +
                                                (int64_t)i * p.ldc + j);
    }
}
template <int OUT, class Raw>
__device__ __forceinline__ f32x4 c_from_raw(const Raw &w) {
    if constexpr (OUT == DT_F32) {
        return __builtin_bit_cast(f32x4, w);
    } else {
        return f32x4{from_out16<OUT>(lo16(w[0])), from_out16<OUT>(hi16(w[0])),
                     from_out16<OUT>(lo16(w[1])), from_out16<OUT>(hi16(w[1]))};
    }
}

// CADDED: the linear part of the epilogue is already in v -- C for the plain
// epilogue, alpha * sum + beta * C + bias for the extended one (both epilogue
// paths load these for a whole row block ahead of its stores); only the
// activation, rounding, satf and store remain.
template <int OUT, bool FULL, bool EPI, bool CADDED = false>
__device__ __forceinline__ void finish4(const Params &p, int i, int j, f32x4 v) {
    const int nval = FULL ? 4 : min(p.N - j, 4);
    if (!FULL && (i >= p.M || nval <= 0)) return;
    if constexpr (OUT < 0) {
        float *w = p.ws + ((int64_t)blockIdx.z * p.M + i) * p.N + j;
        if (FULL) {
            *reinterpret_cast<f32x4 *>(w) = v;
        } else {
            for (int e = 0; e < nval; ++e) w[e] = v[e];
        }
        return;
    } else if constexpr (OUT == DT_I32) {
        // int32: the accumulators hold the exact sum (or its value modulo
        // 2^32 beyond 2^17 products); + C in 64 bits, then wrap or clamp
        const i32x4 sv = __builtin_bit_cast(i32x4, v);
        int64_t t[4] = {sv[0], sv[1], sv[2], sv[3]};
        if (p.C) {
            const int32_t *cp = reinterpret_cast<const int32_t *>(p.C);
            if (FULL) {
                const i32x4 c = *reinterpret_cast<const i32x4 *>(cp + (int64_t)i * p.ldc + j);
#pragma unroll
                for (int e = 0; e < 4; ++e) t[e] += c[e];
            } else {
                for (int e = 0; e < nval; ++e)
                    t[e] += cp[p.c_col ? (int64_t)(j + e) * p.ldc + i : (int64_t)i * p.ldc + j + e];
            }
        }
        i32x4 o;
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = to_int32(t[e], p.satf);
        int32_t *d = reinterpret_cast<int32_t *>(p.D) + (int64_t)i * p.ldd + j;
        if (FULL) {
            *reinterpret_cast<i32x4 *>(d) = o;
        } else {
            for (int e = 0; e < nval; ++e) d[e] = o[e];
        }
    } else {
        // C(i, j..j+3): one vector load when FULL (then C is row-major)
        auto c4 = [&]() {
            f32x4 c;
            if constexpr (OUT == DT_F32) {
                const float *cp = reinterpret_cast<const float *>(p.C) + (int64_t)i * p.ldc + j;
                c = *reinterpret_cast<const f32x4 *>(cp);
            } else {
                const uint16_t *cp =
                    reinterpret_cast<const uint16_t *>(p.C) + (int64_t)i * p.ldc + j;
                const u32x2 w = *reinterpret_cast<const u32x2 *>(cp);
                c = f32x4{from_out16<OUT>(lo16(w[0])), from_out16<OUT>(hi16(w[0])),
                          from_out16<OUT>(lo16(w[1])), from_out16<OUT>(hi16(w[1]))};
            }
            return c;
        };
        if constexpr (!EPI) {
            if (!CADDED && p.C) {
                if (FULL) {
                    v += c4();
                } else {
                    for (int e = 0; e < nval; ++e) v[e] += load_c(p, i, j + e);
                }
            }
        } else if constexpr (!CADDED) {
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = p.alpha * v[e];
            if (p.C) {
                if (FULL) {
                    v += p.beta * c4();
                } else {
                    for (int e = 0; e < nval; ++e) v[e] += p.beta * load_c(p, i, j + e);
                }
            }
            if (p.bias) {
                if (p.bias_rows) {
                    v += p.bias[i];
                } else if (FULL) {
                    v += *reinterpret_cast<const f32x4 *>(p.bias + j);
                } else {
                    for (int e = 0; e < nval; ++e) v[e] += p.bias[j + e];
                }
            }
            if (p.act != ACT_NONE) {
#pragma unroll
                for (int e = 0; e < 4; ++e) v[e] = activate(v[e], p.act);
            }
        } else if (p.act != ACT_NONE) {
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = activate(v[e], p.act);
        }
        const int64_t off = (int64_t)i * p.ldd + j;
        if constexpr (OUT == DT_F32) {
            if (p.satf) {
#pragma unroll
                for (int e = 0; e < 4; ++e) v[e] = satf_f32(v[e]);
            }
            float *d = reinterpret_cast<float *>(p.D) + off;
            if (FULL) {
                *reinterpret_cast<f32x4 *>(d) = v;
            } else {
                for (int e = 0; e < nval; ++e) d[e] = v[e];
            }
        } else {
            const bool sf = p.satf != 0;
            uint16_t *d = reinterpret_cast<uint16_t *>(p.D) + off;
            if (FULL) {
                *reinterpret_cast<u32x2 *>(d) =
                    u32x2{to_out16<OUT>(v[0], sf) | (to_out16<OUT>(v[1], sf) << 16),
                          to_out16<OUT>(v[2], sf) | (to_out16<OUT>(v[3], sf) << 16)};
            } else {
                for (int e = 0; e < nval; ++e) d[e] = (uint16_t)to_out16<OUT>(v[e], sf);
            }
        }
    }
}

// ------------------------------------------------------------ tile mapping
// XCD-aware renumbering and grouped raster of gemm_address.hpp (raster_tile),
// with the group height and skew the host chose for the call.
__device__ __forceinline__ void map_tile(const Params &p, int w, int &tm, int &tn) {
    raster_tile(w, p.tiles_m, p.tiles_n, p.group_m, p.xcds, p.skew, tm, tn);
}

// ------------------------------------------------------------------ K loop
// Software-pipelined K loop over two LDS stages (cur = t & 1), KS MFMA steps
// per K-tile, operand fragments double-buffered by step parity.  Iteration t:
//   step 0      : store K-tile t+1 (in registers) to LDS[cur^1]
//   step 1      : issue the global loads of K-tile t+2
//   step s < KS-1: read the fragments of step s+1 from LDS[cur]
//   step KS-1   : barrier, then read step 0 of K-tile t+1 from LDS[cur^1]
//   every step  : the MFMAs of step s
// One barrier per K-tile orders this tile's LDS reads before the overwrite
// two tiles later and the stores of tile t+1 before its reads.  The body has
// no branches: past the last K-tile the loads re-read it and the stores and
// reads go to the idle stage.
// The loader of one operand tile: K-contiguous operands load chunks as
// stored; R-contiguous ones are transposed in registers (16-bit: LoaderRC,
// 8-bit: LoaderRC8).  The element-wise path (VEC false) gathers K-contiguous
// chunks by layout (LoaderKC::load_checked; LoaderRC's for 16-bit).
template <class CF, int ROWS, bool KC, bool VEC>
using OperandLoader = typename std::conditional<
    KC || (CF::ES == 1 && !VEC), LoaderKC<ROWS, CF::BK, CF::THREADS, CF::ES>,
    typename std::conditional<CF::ES == 1, LoaderRC8<ROWS, CF::BK, CF::THREADS>,
                              LoaderRC<ROWS, CF::BK, CF::THREADS>>::type>::type;

template <class CF, int IT, bool A_KC, bool B_KC, bool VEC, bool RAGGED>
__device__ __forceinline__ void k_loop(const Params &p, int m0, int n0, int kbeg, int kend,
                                       typename AccT<CF::MF>::type (&acc)[CF::TM][CF::TN],
                                       u32x4 *sA, u32x4 *sB, int tid) {
    constexpr int BM = CF::BM, BN = CF::BN, BK = CF::BK, CH = CF::CH;
    constexpr int MF = CF::MF, TM = CF::TM, TN = CF::TN;
    constexpr int KS = BK / CF::KSTEP;           // MFMA steps per K-tile
    constexpr int KCH = CF::KSTEP * CF::ES / 16;  // 16-byte LDS chunks per MFMA step
    static_assert(KS % 2 == 0 && KS >= 2, "fragment slots alternate across K-tiles; the"
                  " store and barrier steps are distinct");
    constexpr int FC = CF::FC;  // 16-byte chunks per lane and operand fragment
    using LA = OperandLoader<CF, BM, A_KC, VEC>;
    using LB = OperandLoader<CF, BN, B_KC, VEC>;

    const int nk = kend > kbeg ? (kend - kbeg + BK - 1) / BK : 0;
    if (nk <= 0) return;

    LA la;
    LB lb;
    la.init(tid, p.lda, m0, p.M);
    lb.init(tid, p.ldb, n0, p.N);
    const __amdgpu_buffer_rsrc_t ra =
        __builtin_amdgcn_make_buffer_rsrc((void *)p.A, (short)0, (int)p.a_bytes, 0x00020000);
    const __amdgpu_buffer_rsrc_t rb =
        __builtin_amdgcn_make_buffer_rsrc((void *)p.B, (short)0, (int)p.b_bytes, 0x00020000);
    auto gload = [&](int kt) {
        const int k0 = kbeg + kt * BK;
        if constexpr (VEC) {
            la.template load<RAGGED>(ra, k0, p.lda, kend);
            lb.template load<RAGGED>(rb, k0, p.ldb, kend);
            if constexpr (RAGGED) {  // only the prologue's stores use this directly
                la.mask(k0, kend);
                lb.mask(k0, kend);
            }
        } else {
            la.template load_checked<!A_KC>(p.A, p.lda, m0, k0, p.M, kend, tid);
            lb.template load_checked<!B_KC>(p.B, p.ldb, n0, k0, p.N, kend, tid);
        }
    };

    // Per-lane LDS byte offsets of each fragment at step 0; step s XORs in
    // s*KCH chunks (the chunk bits of s and of the lane never overlap).
    // Lane l holds chunks lg * FC + c, c < FC, of each step, lg = l / MF
    // (16x16 with one chunk: kc_group16(l / 16)); with FC = 2 the first of
    // them is even, so chunk c sits at offset ^ 16*c.
    static_assert(FC == 1 || FC == 2, "fragment chunks");
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave / CF::WAVES_N, wn = wave % CF::WAVES_N;
    const int lg = (MF == 16 && FC == 1) ? kc_group16(lane / MF) : lane / MF;
    uint32_t a_off[TM], b_off[TN];
#pragma unroll
    for (int i = 0; i < TM; ++i) {
        const int r = wm * CF::WTM + i * MF + (lane & (MF - 1));
        a_off[i] = (uint32_t)(r * CH + ((lg * FC) ^ swz(r))) * 16u;
    }
#pragma unroll
    for (int j = 0; j < TN; ++j) {
        const int r = wn * CF::WTN + j * MF + (lane & (MF - 1));
        b_off[j] = (uint32_t)(r * CH + ((lg * FC) ^ swz(r))) * 16u;
    }

    // With two chunks per fragment (fp8) the double-buffered fragments no
    // longer fit next to the accumulators at two waves per SIMD, so the A
    // fragments are single-buffered: A row i of the next step is read right
    // after the last MFMA of row i in this step (B stays double-buffered).
    constexpr bool A1 = FC == 2;
    u32x4 fa[A1 ? 1 : 2][TM][FC], fb[2][TN][FC];
    // fragment f (A fragments first, then B) of step ks into slot sl
    auto read_one = [&](int buf, auto ks_tag, auto sl_tag, auto f_tag) {
        constexpr int ks = decltype(ks_tag)::value, sl = decltype(sl_tag)::value;
        constexpr int f = decltype(f_tag)::value;
        constexpr uint32_t kx = (uint32_t)(ks * KCH * 16);
        Unroll<0, FC>::run([&](auto c_tag) {
            constexpr int c = decltype(c_tag)::value;
            constexpr uint32_t cx = kx ^ (uint32_t)(16 * c);
            if constexpr (f < TM) {
                const char *ab = reinterpret_cast<const char *>(sA + buf * BM * CH);
                fa[A1 ? 0 : sl][f][c] = *reinterpret_cast<const u32x4 *>(ab + (a_off[f] ^ cx));
            } else {
                const char *bb = reinterpret_cast<const char *>(sB + buf * BN * CH);
                fb[sl][f - TM][c] = *reinterpret_cast<const u32x4 *>(bb + (b_off[f - TM] ^ cx));
            }
        });
    };
    auto mfma_one = [&](auto sl_tag, auto m_tag) {
        constexpr int sl = decltype(sl_tag)::value, m = decltype(m_tag)::value;
        constexpr int i = m / TN, j = m % TN;
        // B fragment as the MFMA's first operand: the instruction then forms
        // the transposed tile, whose rows (D columns) land in consecutive
        // accumulator registers of one lane (see acc_col)
        if constexpr (MF == 32)
            acc[i][j] = mfma32<IT, FC>(fb[sl][j], fa[A1 ? 0 : sl][i], acc[i][j]);
        else
            acc[i][j] = mfma16<IT, FC>(fb[sl][j], fa[A1 ? 0 : sl][i], acc[i][j]);
    };
    auto store_one = [&](int buf, auto w_tag) {
        constexpr int w = decltype(w_tag)::value;
        if constexpr (w < LA::NSTORE)
            la.template store_one<w>(sA + buf * BM * CH, tid);
        else
            lb.template store_one<w - LA::NSTORE>(sB + buf * BN * CH, tid);
    };
    auto load_one = [&](int k0, auto g_tag) {
        constexpr int g = decltype(g_tag)::value;
        if constexpr (g < LA::NLOAD)
            la.template load_one<g, RAGGED>(ra, k0, p.lda, kend);
        else
            lb.template load_one<g - LA::NLOAD, RAGGED>(rb, k0, p.ldb, kend);
    };

    // prologue: K-tile 0 in LDS[0], K-tile 1 in registers, step 0 fragments
    gload(0);
    la.store(sA, tid);
    lb.store(sB, tid);
    gload(nk > 1 ? 1 : 0);
    __syncthreads();
    Unroll<0, TM + TN>::run([&](auto f) {
        read_one(0, std::integral_constant<int, 0>{}, std::integral_constant<int, 0>{}, f);
    });

    constexpr int NM = TM * TN, NR = TM + TN;
    constexpr int NW = LA::NSTORE + LB::NSTORE;
    // Store schedule: the NW stores of K-tile t+1 are spread evenly over the
    // MFMA slots of steps 0..KS-2 (slot s = step*NM + m), A stores first.  A
    // K-contiguous operand's load of K-tile t+2 follows the store that frees
    // its registers; an R-contiguous operand's block is reloaded right after
    // the last of its 8 (transposing) stores.
    constexpr int NSLOT = (KS - 1) * NM;
    auto store_slot = [](int w) { return w * NSLOT / NW; };
    for (int t = 0; t < nk; ++t) {
        const int cur = t & 1;
        const int k_next = kbeg + min(t + 2, nk - 1) * BK;  // K-tile being loaded
        if constexpr (!VEC) {
            // element-wise path: stores and loads as plain blocks
            la.store(sA + (cur ^ 1) * BM * CH, tid);
            lb.store(sB + (cur ^ 1) * BN * CH, tid);
            gload(min(t + 2, nk - 1));
        } else if constexpr (RAGGED) {
            const int k_st = kbeg + min(t + 1, nk - 1) * BK;  // K-tile stored this iteration
            if (k_st + BK > kend) {  // only the last K-tile is ragged (uniform branch)
                la.mask(k_st, kend);
                lb.mask(k_st, kend);
            }
        }
        Unroll<0, KS>::run([&](auto ks_tag) {
            constexpr int ks = decltype(ks_tag)::value;
            constexpr int sl = ks & 1;
            if constexpr (ks == KS - 1) {
                // every LDS read of this K-tile and store of the next is done
                __syncthreads();
                __builtin_amdgcn_sched_barrier(0);
            }
            // One MFMA, then the stores and loads scheduled in its slot, then
            // its share of the next step's fragment reads, in source order
            // (the fences keep the compiler from regrouping them).
            Unroll<0, NM>::run([&](auto m_tag) {
                constexpr int m = decltype(m_tag)::value;
                constexpr int slot = ks * NM + m;
                mfma_one(std::integral_constant<int, sl>{}, m_tag);
                if constexpr (VEC) {
                    Unroll<0, NW>::run([&](auto w_tag) {
                        constexpr int w = decltype(w_tag)::value;
                        if constexpr (w * NSLOT / NW == slot) {
                            store_one(cur ^ 1, w_tag);
                            // a block's loads follow its last store (K-contiguous:
                            // one store and one load per block)
                            if constexpr (w < LA::NSTORE) {
                                constexpr int S = LA::SPB, L = LA::LPB;
                                if constexpr (w % S == S - 1)
                                    Unroll<(w / S) * L, (w / S + 1) * L>::run(
                                        [&](auto g) { load_one(k_next, g); });
                            } else {
                                constexpr int wb = w - LA::NSTORE;
                                constexpr int S = LB::SPB, L = LB::LPB;
                                if constexpr (wb % S == S - 1)
                                    Unroll<LA::NLOAD + (wb / S) * L, LA::NLOAD + (wb / S + 1) * L>::run(
                                        [&](auto g) { load_one(k_next, g); });
                            }
                        }
                    });
                }
                // the next step's fragments in the order that step first uses
                // them (A row 0, then every B column, then the other A rows:
                // its first MFMAs need A0 and all of B at once), one per MFMA
                // from the start of the step, or spread evenly when there are
                // more fragments than MFMAs
                auto read_next = [&](auto f) {
                    if constexpr (ks + 1 < KS)
                        read_one(cur, std::integral_constant<int, ks + 1>{},
                                 std::integral_constant<int, sl ^ 1>{}, f);
                    else
                        read_one(cur ^ 1, std::integral_constant<int, 0>{},
                                 std::integral_constant<int, 0>{}, f);
                };
                if constexpr (A1) {
                    // B column m after MFMA m (m < TN); A row i after its last MFMA
                    if constexpr (m < TN) read_next(std::integral_constant<int, TM + m>{});
                    if constexpr (m % TN == TN - 1)
                        read_next(std::integral_constant<int, m / TN>{});
                } else {
                    constexpr int r_lo = NR <= NM ? (m < NR ? m : NR) : m * NR / NM;
                    constexpr int r_hi = NR <= NM ? (m < NR ? m + 1 : NR) : (m + 1) * NR / NM;
                    Unroll<r_lo, r_hi>::run([&](auto q_tag) {
                        constexpr int q = decltype(q_tag)::value;
                        constexpr int fid = (q == 0) ? 0 : (q <= TN ? TM + q - 1 : q - TN);
                        read_next(std::integral_constant<int, fid>{});
                    });
                }
                __builtin_amdgcn_sched_barrier(0);
            });
        });
    }
    (void)store_slot;
}

// ------------------------------------------------------ K loop, LDS DMA
// The large tiles' K loop on gfx950's direct global -> LDS loads
// (buffer_load_dwordx4 ... lds): no operand passes through registers on its
// way to LDS, so there is no staging, no ds_write and no in-register
// transpose.  Each operand keeps its storage order in LDS:
//   K-contiguous (row-major A, column-major B): [rows][BK] in 16-byte chunks,
//     read with ds_read_b128 (one chunk per lane and MFMA operand, two for
//     the fp8 MFMAs); 16-bit and 8-bit values alike (rows of 128 bytes);
//   R-contiguous (row-major B, column-major A): [BK][rows], read with the
//     transposing ds_read_b64_tr_b16 (two per lane and MFMA operand) or, for
//     8-bit values, ds_read_b64_tr_b8 (two per 16-byte chunk; 32x32 MFMA).
// The XOR swizzles (gemm_address.hpp) are applied on the global side: lane l
// of a DMA instruction fills LDS chunk q0 + l, so it fetches the chunk that
// belongs in that slot.
//
// Two LDS stages.  Iteration t computes K-tile t from stage t & 1; its last
// MFMA step starts with: wait for this wave's DMA of tile t+1, barrier (every
// wave's DMA of tile t+1 has landed and every wave has finished reading
// stage t & 1), then the DMA of tile t+2 into stage t & 1 is issued across
// that step's MFMAs, which also read tile t+1's first fragments.  So a
// tile's loads have one full K-tile of MFMA work to land in.  In the last
// two iterations there is no tile t+2: the same DMA instructions then load
// the last tile again into a 1 KiB sink no one reads, which keeps the loop
// body free of branches (a branch there made the compiler shuffle the
// accumulators between register files).  The compiler does not order LDS
// DMA against LDS reads; the explicit vmcnt wait and the barrier do.
//
// A ragged last K-tile (k >= kend inside it) is loaded with clamped
// addresses, then its k >= kend part is zeroed in LDS before it is read.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    // gfx9 s_waitcnt: vmcnt in bits 3:0 and 15:14, expcnt 6:4 (7: no wait),
    // lgkmcnt 11:8 (15: no wait)
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

typedef short s16x4 __attribute__((ext_vector_type(4)));
#define LIBGEMM_LDS __attribute__((address_space(3)))

__device__ __forceinline__ u32x2 ds_read_tr16(const char *p) {
    const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LIBGEMM_LDS s16x4 *)(p));
    return __builtin_bit_cast(u32x2, v);
}

__device__ __forceinline__ u32x2 ds_read_tr8(const char *p) {
    const i32x2 v = __builtin_amdgcn_ds_read_tr8_b64_v2i32((LIBGEMM_LDS i32x2 *)(p));
    return __builtin_bit_cast(u32x2, v);
}

__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t rsrc, char *lds_dst, uint32_t voff,
                                      uint32_t soff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (LIBGEMM_LDS void *)lds_dst, 16, (int)voff,
                                             (int)soff, 0, 0);
}

// One operand's DMA for the K loop: ROWS x BK tile of ES-byte values (16-bit
// or 8-bit), KC or R-contiguous storage, NWAVES waves sharing the tile's
// 1 KiB DMA blocks.
template <int ROWS, int BK, int NWAVES, int MF, bool KC, bool CLAMPK, int ES = 2>
struct DmaOperand {
    static constexpr int BYTES = ROWS * BK * ES;
    static constexpr int NI = BYTES / 1024 / NWAVES;  // DMA instructions per wave
    static_assert(BYTES % (1024 * NWAVES) == 0, "1 KiB DMA blocks per wave");
    static constexpr int EPC = 16 / ES;        // elements per 16-byte chunk
    static constexpr int CH = BK * ES / 16;    // KC: chunks per row
    static constexpr int CHR = ROWS * ES / 16; // RC: chunks per k-row
    static_assert(KC || CHR >= 16, "the R-contiguous swizzles need 16 chunks per k-row");
    uint32_t voff[NI];  // byte offset at k0 = 0 (CLAMPK: without the k part)
    int kpos[NI];       // CLAMPK: k position of the chunk (KC) or the k-row (RC)

    __device__ __forceinline__ void init(int lane, int wave, int r0, int R, int64_t ld) {
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            const int q = (wave * NI + i) * 64 + lane;
            int a, c;
            if constexpr (KC) {
                dma_kc_source(q, CH, a, c);  // a = row, chunk c holds k = EPC*c..
                kpos[i] = EPC * c;
                voff[i] =
                    (uint32_t)kc_chunk_offset(r0 + a, CLAMPK ? 0 : EPC * c, R, 1, ld, ES, false);
            } else if constexpr (ES == 2) {
                dma_rc_source(q, CHR, MF, a, c);  // a = k-row, rows 8c..8c+7
                kpos[i] = a;
                voff[i] = (uint32_t)rc_chunk_offset(r0 + 8 * c, CLAMPK ? 0 : a, R, 1, ld, false);
            } else {
                dma_rc8_source(q, CHR, a, c);  // a = k-row, rows 16c..16c+15
                kpos[i] = a;
                voff[i] = (uint32_t)rc8_chunk_offset(r0 + 16 * c, CLAMPK ? 0 : a, R, 1, ld, false);
            }
        }
    }

    // DMA instruction i of this wave for the K-tile at k0 into the stage at
    // lds, or into the 1 KiB block sink when the stage is not to be written
    __device__ __forceinline__ void issue(__amdgpu_buffer_rsrc_t rsrc, char *lds, char *sink,
                                          bool real, int wave, int i, int k0, int64_t ld,
                                          int kend) const {
        char *dst = real ? lds + (wave * NI + i) * 1024 : sink;
        if constexpr (KC) {
            if constexpr (CLAMPK)
                dma16(rsrc, dst, voff[i] + (uint32_t)kc_k_offset(k0 + kpos[i], kend, ES), 0u);
            else
                dma16(rsrc, dst, voff[i], (uint32_t)k0 * (uint32_t)ES);
        } else {
            constexpr uint32_t es = ES;
            if constexpr (CLAMPK)
                dma16(rsrc, dst, voff[i] + (uint32_t)imin(k0 + kpos[i], kend - 1) * (uint32_t)ld * es,
                      0u);
            else
                dma16(rsrc, dst, voff[i], (uint32_t)k0 * (uint32_t)ld * es);
        }
    }

    // zero k >= kvalid of the tile in LDS (the ragged last K-tile), threads
    // tid of nthreads
    __device__ __forceinline__ static void zero_tail(char *lds, int kvalid, int tid, int nthreads) {
        if constexpr (KC) {
            for (int q = tid; q < ROWS * CH; q += nthreads) {
                const int r = q / CH, c = q % CH;  // logical chunk c: k = EPC*c..
                const int keep = kvalid - EPC * c;
                if (keep >= EPC) continue;
                u32x4 *dst = reinterpret_cast<u32x4 *>(lds + (r * CH + (c ^ swz_kc(r))) * 16);
                const u32x4 kept = ES == 2 ? keep_first(*dst, keep) : keep_first_bytes(*dst, keep);
                *dst = keep <= 0 ? u32x4{0u, 0u, 0u, 0u} : kept;
            }
        } else {
            for (int q = tid; q < (BK - kvalid) * CHR; q += nthreads)
                reinterpret_cast<u32x4 *>(lds + (kvalid + q / CHR) * ROWS * ES)[q % CHR] =
                    u32x4{0u, 0u, 0u, 0u};
        }
    }
};

template <class CF, int IT, bool A_KC, bool B_KC, bool RAGGED>
__device__ __forceinline__ void dma_k_loop(const Params &p, int m0, int n0, int kbeg, int kend,
                                           typename AccT<CF::MF>::type (&acc)[CF::TM][CF::TN],
                                           char *lds, int tid) {
    constexpr int BM = CF::BM, BN = CF::BN, BK = CF::BK;
    constexpr int MF = CF::MF, TM = CF::TM, TN = CF::TN;
    constexpr int NWAVES = CF::WAVES_M * CF::WAVES_N;
    constexpr int ES = CF::ES, FC = CF::FC;
    constexpr int KS = BK / CF::KSTEP;            // MFMA steps per K-tile
    constexpr int KCH = CF::KSTEP * ES / 16;      // 16-byte chunks per step (KC reads)
    static_assert((ES == 2 && FC == 1) || (ES == 1 && (MF == 32 || (A_KC && B_KC))),
                  "16-bit operands, or 8-bit ones (R-contiguous: the 32x32 MFMA)");
    static_assert(FC == 1 || FC == 2, "fragment chunks");
    static_assert(BK * ES == 128, "LDS rows of 128 bytes (KC layout)");
    static_assert(KS % 2 == 0, "fragment slots alternate across K-tiles");
    // B_REG (row-major B with row-major A, one wave per SIMD): B is loaded
    // into registers and transposed on its way to LDS by LoaderRC, so LDS
    // holds it K-contiguous like A; with one wave per SIMD a transposed LDS
    // read of B costs more than that register transpose (measured).  With
    // two waves per SIMD, and with column-major A, B takes the transposed
    // reads.
    constexpr bool B_REG = A_KC && !B_KC && NWAVES == 4;
    constexpr bool B_KCL = B_KC || B_REG;  // B's LDS tile is K-contiguous
    using DA = DmaOperand<BM, BK, NWAVES, MF, A_KC, RAGGED, ES>;
    using DB = DmaOperand<BN, BK, NWAVES, MF, B_KCL, RAGGED, ES>;
    using LB = LoaderRC<BN, B_REG ? BK : 64, CF::THREADS>;  // (unused unless B_REG)
    constexpr int SA = DA::BYTES, SB = DB::BYTES;  // bytes per stage
    char *const ldsA = lds, *const ldsB = lds + 2 * SA;

    const int nk = kend > kbeg ? (kend - kbeg + BK - 1) / BK : 0;
    if (nk <= 0) return;

    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / CF::WAVES_N, wn = wave % CF::WAVES_N;
    DA da;
    DB db;
    LB lb;
    da.init(lane, wave, m0, p.M, p.lda);
    if constexpr (B_REG) lb.init(tid, p.ldb, n0, p.N);
    else db.init(lane, wave, n0, p.N, p.ldb);
    const __amdgpu_buffer_rsrc_t ra =
        __builtin_amdgcn_make_buffer_rsrc((void *)p.A, (short)0, (int)p.a_bytes, 0x00020000);
    const __amdgpu_buffer_rsrc_t rb =
        __builtin_amdgcn_make_buffer_rsrc((void *)p.B, (short)0, (int)p.b_bytes, 0x00020000);
    char *const sink = lds + 2 * (SA + SB);  // 1 KiB that no one reads
    // g-th DMA instruction of this wave for the tile at k0 into stage (real)
    // or into the sink
    auto dma_one = [&](int g, int stage, int k0, bool real) {
        if (g < DA::NI) da.issue(ra, ldsA + stage * SA, sink, real, wave, g, k0, p.lda, kend);
        else db.issue(rb, ldsB + stage * SB, sink, real, wave, g - DA::NI, k0, p.ldb, kend);
    };
    auto zero_ragged = [&](int stage, int k0) {  // the tile at k0 is the ragged last one
        DA::zero_tail(ldsA + stage * SA, kend - k0, tid, CF::THREADS);
        if constexpr (!B_REG) DB::zero_tail(ldsB + stage * SB, kend - k0, tid, CF::THREADS);
    };
    // B_REG: the register loads of B's tile at k0, and its transposing
    // stores into a stage (k >= kend masked to zero in RAGGED kernels; the
    // mask is a no-op on full tiles and keeps the loop free of branches)
    auto b_store = [&](int stage, int k0, auto w_tag) {
        constexpr int w = decltype(w_tag)::value;
        if constexpr (RAGGED && w == 0) lb.mask(k0, kend);
        lb.template store_one<w>(reinterpret_cast<u32x4 *>(ldsB + stage * SB), tid);
    };

    // per-lane LDS byte offsets of each fragment at step 0, stage 0 (KC: lane
    // l holds chunks lg * FC + c, c < FC, of each step, as in k_loop; the
    // 16x16 order of kc_group16 only when both operands are read K-contiguous,
    // as the transposed reads take lane group g to k-group g)
    const int lg = (MF == 16 && FC == 1 && A_KC && B_KCL) ? kc_group16(lane / MF) : lane / MF;
    uint32_t a_off[TM], b_off[TN];
#pragma unroll
    for (int i = 0; i < TM; ++i) {
        const int rb0 = wm * CF::WTM + i * MF;
        if constexpr (A_KC) {
            const int r = rb0 + (lane & (MF - 1));
            a_off[i] = (uint32_t)(r * DA::CH + ((lg * FC) ^ swz_kc(r))) * 16u;
        } else {
            a_off[i] = ES == 2 ? (uint32_t)tr_read_offset(lane, MF, 0, 0, rb0, BM * 2)
                               : (uint32_t)tr8_read_offset(lane, FC, 0, CF::KSTEP, 0, 0, rb0, BM);
        }
    }
#pragma unroll
    for (int j = 0; j < TN; ++j) {
        const int rb0 = wn * CF::WTN + j * MF;
        if constexpr (B_KCL) {
            const int r = rb0 + (lane & (MF - 1));
            b_off[j] = (uint32_t)(r * DB::CH + ((lg * FC) ^ swz_kc(r))) * 16u;
        } else {
            b_off[j] = ES == 2 ? (uint32_t)tr_read_offset(lane, MF, 0, 0, rb0, BN * 2)
                               : (uint32_t)tr8_read_offset(lane, FC, 0, CF::KSTEP, 0, 0, rb0, BN);
        }
    }

    // Two-chunk fragments (fp8): A single-buffered, as in k_loop (A row i of
    // the next step is read right after the last MFMA of row i in this step)
    constexpr bool A1 = FC == 2;
    u32x4 fa[A1 ? 1 : 2][TM][FC], fb[2][TN][FC];
    // fragment f (A fragments first, then B) of step ks from stage st into slot sl
    auto read_one = [&](int st, auto ks_tag, auto sl_tag, auto f_tag) {
        constexpr int ks = decltype(ks_tag)::value, sl = decltype(sl_tag)::value;
        constexpr int f = decltype(f_tag)::value;
        constexpr bool isA = f < TM;
        constexpr bool kc = isA ? A_KC : B_KCL;
        constexpr int RB = (isA ? BM : BN) * ES;  // R-contiguous: bytes per k-row
        const char *base;
        uint32_t off;
        if constexpr (isA) {
            base = ldsA + st * SA;
            off = a_off[f];
        } else {
            base = ldsB + st * SB;
            off = b_off[f - TM];
        }
        u32x4 v[FC];
        if constexpr (kc) {
            // K-contiguous: chunks ks*KCH + (lane/MF)*FC + c of the row; the
            // step's chunk bits, the lane's and c's never overlap, so XOR adds
            // them
            Unroll<0, FC>::run([&](auto c_tag) {
                constexpr int c = decltype(c_tag)::value;
                constexpr uint32_t cx = (uint32_t)(ks * KCH * 16) ^ (uint32_t)(16 * c);
                v[c] = *reinterpret_cast<const u32x4 *>(base + (off ^ cx));
            });
        } else if constexpr (ES == 2) {
            // R-contiguous: the step and half move whole k-rows (k % 4 and
            // bit 3 of k, which the swizzle uses, are the lane's own)
            constexpr uint32_t kstep_rows = MF == 32 ? 16 : 32;
            const u32x2 lo = ds_read_tr16(base + off + ks * kstep_rows * RB);
            const u32x2 hi = ds_read_tr16(base + off + (ks * kstep_rows + 4) * RB);
            v[0] = u32x4{lo[0], lo[1], hi[0], hi[1]};
        } else {
            // R-contiguous 8-bit: chunk c's halves are k-rows 16c and 16c + 8
            // on from the step's; the swizzle uses k % 8, the lane's own
            Unroll<0, FC>::run([&](auto c_tag) {
                constexpr int c = decltype(c_tag)::value;
                constexpr uint32_t k0 = (uint32_t)(ks * CF::KSTEP + 16 * c);
                const u32x2 lo = ds_read_tr8(base + off + k0 * RB);
                const u32x2 hi = ds_read_tr8(base + off + (k0 + 8) * RB);
                v[c] = u32x4{lo[0], lo[1], hi[0], hi[1]};
            });
        }
        Unroll<0, FC>::run([&](auto c_tag) {
            constexpr int c = decltype(c_tag)::value;
            if constexpr (isA) fa[A1 ? 0 : sl][f][c] = v[c];
            else fb[sl][f - TM][c] = v[c];
        });
    };
    auto mfma_one = [&](auto sl_tag, auto m_tag) {
        constexpr int sl = decltype(sl_tag)::value, m = decltype(m_tag)::value;
        constexpr int i = m / TN, j = m % TN;
        constexpr int sa = A1 ? 0 : sl;
        if constexpr (MF == 32) acc[i][j] = mfma32<IT, FC>(fb[sl][j], fa[sa][i], acc[i][j]);
        else acc[i][j] = mfma16<IT, FC>(fb[sl][j], fa[sa][i], acc[i][j]);
    };

    // prologue: tiles 0 and 1 in flight, wait for tile 0, its step-0
    // fragments (B_REG: B of tile 0 stored; B of tile 1 loaded into the
    // registers before A's DMA of tile 1, the order the loop keeps)
    constexpr int NDMA = DA::NI + (B_REG ? 0 : DB::NI);  // DMA instructions per wave and tile
    constexpr int NBL = B_REG ? LB::NLOAD : 0;             // B register loads per thread and tile
#pragma unroll
    for (int g = 0; g < NDMA; ++g) dma_one(g, 0, kbeg, true);
    if constexpr (B_REG) {
        lb.template load<RAGGED>(rb, kbeg, p.ldb, kend);
        Unroll<0, LB::NSTORE>::run([&](auto w) { b_store(0, kbeg, w); });
        lb.template load<RAGGED>(rb, kbeg + min(1, nk - 1) * BK, p.ldb, kend);
    }
    if (nk > 1) {
#pragma unroll
        for (int g = 0; g < NDMA; ++g) dma_one(g, 1, kbeg + BK, true);
        wait_vmcnt<NDMA + NBL>();
    } else {
        wait_vmcnt<NBL>();
    }
    __syncthreads();
    if constexpr (RAGGED) {
        if (kbeg + BK > kend) {
            zero_ragged(0, kbeg);
            __syncthreads();
        }
    }
    Unroll<0, TM + TN>::run([&](auto f) {
        read_one(0, std::integral_constant<int, 0>{}, std::integral_constant<int, 0>{}, f);
    });

    constexpr int NM = TM * TN, NR = TM + TN;
    for (int t = 0; t < nk; ++t) {
        const int cur = t & 1;
        // the DMA of tile t+2; past the last tile the loads go to the sink
        // (from the last tile's addresses), so the loop body has no branch
        const bool more = t + 2 < nk;
        const int k_pre = kbeg + min(t + 2, nk - 1) * BK;
        const int k_next = kbeg + min(t + 1, nk - 1) * BK;  // B_REG: the tile stored in step 0
        Unroll<0, KS>::run([&](auto ks_tag) {
            constexpr int ks = decltype(ks_tag)::value;
            constexpr int sl = ks & 1;
            if constexpr (ks == KS - 1) {
                // tile t+1 has landed everywhere; stage cur is no longer read
                // (B_REG: B's loads of tile t+2, issued in step 0, stay in
                // flight; the counter retires in order)
                wait_vmcnt<NBL>();
                __syncthreads();
                if constexpr (RAGGED) {
                    if (t + 1 < nk && kbeg + (t + 2) * BK > kend) {
                        zero_ragged(cur ^ 1, kbeg + (t + 1) * BK);
                        __syncthreads();
                    }
                }
                __builtin_amdgcn_sched_barrier(0);
            }
            // one MFMA, then its share of the next step's fragment reads (in
            // the order that step first uses them: A row 0, every B column,
            // then the other A rows) and, in the last step, of the DMA of
            // tile t+2
            Unroll<0, NM>::run([&](auto m_tag) {
                constexpr int m = decltype(m_tag)::value;
                mfma_one(std::integral_constant<int, sl>{}, m_tag);
                if constexpr (ks == KS - 1) {
                    Unroll<0, NDMA>::run([&](auto g_tag) {
                        constexpr int g = decltype(g_tag)::value;
                        if constexpr (g * NM / NDMA == m) dma_one(g, cur, k_pre, more);
                    });
                }
                if constexpr (B_REG && ks == 0) {
                    // B of tile t+1 (loaded one tile ago) into its stage, one
                    // store per MFMA; then the loads of tile t+2 into the
                    // freed registers (past the last tile: the last one again)
                    if constexpr (m < LB::NSTORE)
                        b_store(cur ^ 1, k_next, std::integral_constant<int, m>{});
                    else if constexpr (m - LB::NSTORE < LB::NLOAD)
                        lb.template load_one<m - LB::NSTORE, RAGGED>(rb, k_pre, p.ldb, kend);
                }
                auto read_next = [&](auto fq) {
                    if constexpr (ks + 1 < KS)
                        read_one(cur, std::integral_constant<int, ks + 1>{},
                                 std::integral_constant<int, sl ^ 1>{}, fq);
                    else
                        read_one(cur ^ 1, std::integral_constant<int, 0>{},
                                 std::integral_constant<int, sl ^ 1>{}, fq);
                };
                if constexpr (A1) {
                    // B column m after MFMA m (m < TN); A row i after its last MFMA
                    if constexpr (m < TN) read_next(std::integral_constant<int, TM + m>{});
                    if constexpr (m % TN == TN - 1)
                        read_next(std::integral_constant<int, m / TN>{});
                } else {
                    constexpr int r_lo = NR <= NM ? (m < NR ? m : NR) : m * NR / NM;
                    constexpr int r_hi = NR <= NM ? (m < NR ? m + 1 : NR) : (m + 1) * NR / NM;
                    Unroll<r_lo, r_hi>::run([&](auto q_tag) {
                        constexpr int q = decltype(q_tag)::value;
                        constexpr int fid = (q == 0) ? 0 : (q <= TN ? TM + q - 1 : q - TN);
                        read_next(std::integral_constant<int, fid>{});
                    });
                }
                __builtin_amdgcn_sched_barrier(0);
            });
        });
    }
}

// ---------------------------------------------------------------- epilogue
// Register group g (4 consecutive D columns) of one accumulator tile.  AGPR:
// the accumulators live in the AGPRs (kernels with 256 of them per lane);
// each group is then moved to VGPRs right where the epilogue uses it
// (v_accvgpr_read, a register move), so the 256 accumulators are never all
// needed in VGPRs at once.
__device__ __forceinline__ float agpr_read(float a) {
    float v;
    asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(v) : "a"(a));
    return v;
}

template <bool AGPR, class T>
__device__ __forceinline__ f32x4 acc_group(const T &t, int g) {
    if constexpr (AGPR)
        return f32x4{agpr_read(t[4 * g]), agpr_read(t[4 * g + 1]), agpr_read(t[4 * g + 2]),
                     agpr_read(t[4 * g + 3])};
    else
        return f32x4{t[4 * g], t[4 * g + 1], t[4 * g + 2], t[4 * g + 3]};
}

// Finish one BM x BN tile from its accumulators: each lane owns 4
// consecutive columns of one row per register group.  smem (SMEM_BYTES of
// LDS) is free for staging: the K loop's reads of it are complete.
// EPIX_OK: interior tiles may take the extended epilogue (fp32 out) in
// registers; otherwise it always goes through the staged loop.
template <class CF, int IT, bool VEC, int SMEM_BYTES, bool AGPR = false, bool EPIX_OK = false>
__device__ __forceinline__ void tile_epilogue(const Params &p,
                                              typename AccT<CF::MF>::type (&acc)[CF::TM][CF::TN],
                                              int m0, int n0, u32x4 *smem, int tid) {
    constexpr int BM = CF::BM, BN = CF::BN;
    constexpr int MF = CF::MF, TM = CF::TM, TN = CF::TN;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave / CF::WAVES_N, wn = wave % CF::WAVES_N;

    // Epilogue.  Each lane owns 4 consecutive columns of one row per register
    // group.  Interior tiles with vector-friendly C/D and the plain epilogue
    // (+C) finish and store those straight from registers (C add, convert,
    // satf, one vector store per group).  Everything else -- edge tiles,
    // split-K slices, unaligned or column-major C, and the extended epilogue
    // (scale, bias, activation) -- stages the tile through LDS one MF-row block
    // at a time and finishes it in a loop that is not unrolled, so the
    // extended arithmetic is instantiated once.  There, groups that lie inside
    // M x N still use vector loads and stores; only groups that cross the
    // edge, or unaligned / column-major C and D, go element by element.
    constexpr int NG = AccT<MF>::N / 4;  // 4-column groups per MFMA tile and lane
    const bool full = (m0 + BM <= p.M) && (n0 + BN <= p.N) && p.cd_vec && p.splits == 1;
    // every tile of a float output (at the M edge rows >= M are skipped, at
    // the N edge groups past N; int8 kernels, whose epilogue holds no C ahead,
    // take interior tiles only: the checks cost them spills)
    const bool ncols = IT == IT_I8 ? full : p.cd_vec && p.splits == 1;
    // (Edge tiles go through the staged loop below, which stores every group
    // inside M x N with vector stores too.  Handling them here, with a bounds
    // check and an element-wise fallback per group, made this unrolled code
    // three times larger: that cost int8 20% (epilogue spills) and the
    // 16384^2 x 1024 shape, 16 tiles per CU, 25%.)
    auto direct = [&](auto out_tag, auto epix_tag) {
        constexpr int OUT = decltype(out_tag)::value;
        // EPIX: the extended epilogue (scale, bias, activation) in registers
        constexpr bool EPIX = decltype(epix_tag)::value;
        // Float outputs load C ahead of the stores, for RB row blocks at a
        // time: a wait for a load also waits for every earlier store, so
        // loads issued between stores serialise them.  RB row blocks of C
        // take at most 64 registers (all of a wave's C when it is 16-bit).
        constexpr bool PRE = OUT != DT_I32;
        constexpr int CW = (OUT == DT_F32) ? 4 : 2;  // registers per 4-column group of C
        constexpr int RB0 = 64 / (TN * NG * CW) < 1 ? 1 : 64 / (TN * NG * CW);
        constexpr int RB = RB0 >= TM ? TM : (TM % RB0 == 0 ? RB0 : 1);
        auto col_of = [&](int j, int g) {
            return n0 + wn * CF::WTN + j * MF + acc_col<MF>(lane, g);
        };
        auto row_of = [&](int i) { return m0 + wm * CF::WTM + i * MF + acc_row<MF>(lane); };
        // EPIX: the bias of the lane's columns, loaded before any store (the
        // same for every row block; a load between stores would wait for them)
        f32x4 bcol[EPIX ? TN : 1][EPIX ? NG : 1];
        if constexpr (EPIX) {
            Unroll<0, TN>::run([&](auto jj) {
                Unroll<0, NG>::run([&](auto gg) {
                    constexpr int j = decltype(jj)::value, g = decltype(gg)::value;
                    const int col = col_of(j, g);
                    bcol[j][g] = (p.bias && !p.bias_rows && col + 4 <= p.N)
                                     ? *reinterpret_cast<const f32x4 *>(p.bias + col)
                                     : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
                });
            });
        }
        Unroll<0, TM / RB>::run([&](auto bb) {
            constexpr int i0 = decltype(bb)::value * RB;
            // raw C bits (fp32: 4 words per group, 16-bit: 2), converted at the store
            using Raw = typename std::conditional<OUT == DT_F32, u32x4, u32x2>::type;
            Raw cpre[RB][TN][NG];
            if constexpr (PRE) {
                Unroll<0, RB>::run([&](auto rr) {
                    Unroll<0, TN>::run([&](auto jj) {
                        Unroll<0, NG>::run([&](auto gg) {
                            constexpr int r = decltype(rr)::value, j = decltype(jj)::value;
                            constexpr int g = decltype(gg)::value;
                            const int row = row_of(i0 + r), col = col_of(j, g);
                            const bool in = row < p.M && col + 4 <= p.N;
                            cpre[r][j][g] = Raw{};
                            if (p.C) cpre[r][j][g] = load_c_raw<OUT>(p, in ? row : 0, in ? col : 0);
                        });
                    });
                });
            }
            // bias by row (a column-major D's transposed problem): one value per row
            float brow[RB];
            if constexpr (EPIX) {
                Unroll<0, RB>::run([&](auto rr) {
                    constexpr int r = decltype(rr)::value;
                    const int row = row_of(i0 + r);
                    brow[r] = (p.bias && p.bias_rows) ? p.bias[row < p.M ? row : 0] : 0.0f;
                });
            }
            Unroll<0, RB>::run([&](auto rr) {
                constexpr int r = decltype(rr)::value, i = i0 + r;
                const int row = row_of(i);
                if constexpr (IT != IT_I8) {
                    if (row >= p.M) return;
                }
                Unroll<0, TN>::run([&](auto jj) {
                    constexpr int j = decltype(jj)::value;
                    Unroll<0, NG>::run([&](auto gg) {
                        constexpr int g = decltype(gg)::value;
                        const int col = col_of(j, g);
                        const f32x4 v = acc_group<AGPR>(acc[i][j], g);
                        if constexpr (IT == IT_I8) {
                            finish4<OUT, true, false>(p, row, col, v);
                        } else if (col + 4 <= p.N) {
                            if constexpr (EPIX) {
                                // alpha * sum + beta * C + bias, then the activation
                                f32x4 x = p.alpha * v;
                                if (p.C) x += p.beta * c_from_raw<OUT>(cpre[r][j][g]);
                                if (p.bias) {
                                    x += p.bias_rows ? f32x4{brow[r], brow[r], brow[r], brow[r]}
                                                     : bcol[j][g];
                                }
                                finish4<OUT, true, true, true>(p, row, col, x);
                            } else {
                                finish4<OUT, true, false, true>(p, row, col,
                                                                v + c_from_raw<OUT>(cpre[r][j][g]));
                            }
                        }
                    });
                });
            });
        });
        // At the N edge, the lane's group that crosses it (column pc, the same
        // in every row the lane holds): gathered from the accumulators by
        // selects, finished element-wise once per row
        if constexpr (IT != IT_I8) {
            if (!full && n0 + BN > p.N) {
                int pc = -1;
                Unroll<0, TN>::run([&](auto jj) {
                    Unroll<0, NG>::run([&](auto gg) {
                        const int c = col_of(decltype(jj)::value, decltype(gg)::value);
                        if (c < p.N && c + 4 > p.N) pc = c;
                    });
                });
                Unroll<0, TM>::run([&](auto ii) {
                    constexpr int i = decltype(ii)::value;
                    f32x4 v = {0.0f, 0.0f, 0.0f, 0.0f};
                    Unroll<0, TN>::run([&](auto jj) {
                        Unroll<0, NG>::run([&](auto gg) {
                            constexpr int j = decltype(jj)::value, g = decltype(gg)::value;
                            if (col_of(j, g) == pc) v = acc_group<AGPR>(acc[i][j], g);
                        });
                    });
                    if (pc >= 0) finish4<OUT, false, EPIX>(p, row_of(i), pc, v);
                });
            }
        }
    };
    // (kernels with element-wise operand loads serve unaligned operands, a
    // slow path anyway: they finish through the staged loop only)
    if constexpr (VEC) {
        using NoX = std::false_type;
        if (ncols && !p.epi) {
            if constexpr (IT == IT_I8) direct(std::integral_constant<int, DT_I32>{}, NoX{});
            else if (p.out_dtype == DT_F32) direct(std::integral_constant<int, DT_F32>{}, NoX{});
            else if (p.out_dtype == DT_F16) direct(std::integral_constant<int, DT_F16>{}, NoX{});
            else direct(std::integral_constant<int, DT_BF16>{}, NoX{});
            return;
        }
        if constexpr (IT != IT_I8 && EPIX_OK) {
            if (ncols && p.epi && p.out_dtype == DT_F32) {
                direct(std::integral_constant<int, DT_F32>{}, std::true_type{});
                return;
            }
        }
    }
    // staged path: one MF-row block per wave at a time in the wave's own LDS
    // region (free: the K loop's last barrier has passed), rows padded
    // against bank conflicts, read back four columns per lane
    {
        constexpr int WTN = CF::WTN;
        constexpr int SROW = WTN + 8;          // floats per staged row
        constexpr int LPR = WTN / 4;           // lanes per staged row
        constexpr int RPP = 64 / LPR;          // rows per pass of the wave
        constexpr int PASSES = MF / RPP;       // passes per row block
        constexpr int QB = PASSES < 8 ? PASSES : 8;  // passes whose loads are in flight together
        static_assert(64 % LPR == 0 && PASSES % QB == 0, "lanes per staged row");
        static_assert(CF::WAVES_M * CF::WAVES_N * MF * SROW * 4 <= SMEM_BYTES,
                      "staging fits in the operand buffers");
        float *stage = reinterpret_cast<float *>(smem) + wave * MF * SROW;
        const int row0 = m0 + wm * CF::WTM, col0 = n0 + wn * WTN;
        const int c4 = (lane % LPR) * 4, gj = col0 + c4;
        const bool gin = gj + 4 <= p.N;
        // group (gi, gj..gj+3) inside M x N with vector-friendly C, D and bias
        auto gfull_at = [&](int gi) { return full || (p.cd_vec && p.splits == 1 && gi < p.M && gin); };
        // Linear part of the epilogue (alpha * sum + beta * C + bias, or sum + C)
        // applied in place to the staged groups that lie inside M x N (the
        // vector groups), with all of a row block's C and bias loads issued
        // before any of its stores: on gfx9 a wait for a load also waits for
        // every earlier store, so loading per group would serialise the
        // stores.  The loads are unconditional (a group outside M x N reads
        // C(0, 0) and discards it), so no branch splits them.  Groups that
        // cross the edge keep the whole epilogue for the finish step.  (int32
        // outputs add C in 64 bits at the store instead.)
        auto linear = [&](auto out_tag, int i) {
            constexpr int OUT = decltype(out_tag)::value;
            f32x4 bcol = {0.0f, 0.0f, 0.0f, 0.0f};
            if (p.epi && p.bias && !p.bias_rows && gin)
                bcol = *reinterpret_cast<const f32x4 *>(p.bias + gj);
#pragma nounroll
            for (int q0 = 0; q0 < PASSES; q0 += QB) {
                // raw C bits (fp32: 4 words, 16-bit: 2), converted after all loads
                u32x4 craw[QB];
                float brow[QB];
                auto row_q = [&](int q) {
                    const int gi = row0 + i * MF + lane / LPR + (q0 + q) * RPP;
                    return gfull_at(gi) ? gi : -1;
                };
                if (p.C) {
                    Unroll<0, QB>::run([&](auto qq) {
                        constexpr int q = decltype(qq)::value;
                        const int gi = row_q(q);
                        const int64_t off = gi < 0 ? 0 : (int64_t)gi * p.ldc + gj;
                        if constexpr (OUT == DT_F32) {
                            craw[q] = *reinterpret_cast<const u32x4 *>(
                                reinterpret_cast<const float *>(p.C) + off);
                        } else {
                            const u32x2 w = *reinterpret_cast<const u32x2 *>(
                                reinterpret_cast<const uint16_t *>(p.C) + off);
                            craw[q] = u32x4{w[0], w[1], 0u, 0u};
                        }
                    });
                }
                if (p.epi && p.bias && p.bias_rows) {
                    Unroll<0, QB>::run([&](auto qq) {
                        constexpr int q = decltype(qq)::value;
                        const int gi = row_q(q);
                        brow[q] = p.bias[gi < 0 ? 0 : gi];
                    });
                }
                Unroll<0, QB>::run([&](auto qq) {
                    constexpr int q = decltype(qq)::value;
                    const int rr = lane / LPR + (q0 + q) * RPP;
                    if (!gfull_at(row0 + i * MF + rr)) return;
                    f32x4 *sp = reinterpret_cast<f32x4 *>(stage + rr * SROW + c4);
                    f32x4 v = *sp;
                    auto c = [&]() {
                        if constexpr (OUT == DT_F32) return __builtin_bit_cast(f32x4, craw[q]);
                        else return f32x4{from_out16<OUT>(lo16(craw[q][0])), from_out16<OUT>(hi16(craw[q][0])),
                                          from_out16<OUT>(lo16(craw[q][1])), from_out16<OUT>(hi16(craw[q][1]))};
                    };
                    if (p.epi) {
#pragma unroll
                        for (int e = 0; e < 4; ++e) v[e] = p.alpha * v[e];
                        if (p.C) v += p.beta * c();
                        if (p.bias) v += p.bias_rows ? f32x4{brow[q], brow[q], brow[q], brow[q]} : bcol;
                    } else if (p.C) {
                        v += c();
                    }
                    *sp = v;
                });
            }
        };
#pragma nounroll
        for (int i = 0; i < TM; ++i) {
            // stage row block i (constant accumulator indices in each case)
            Unroll<0, TM>::run([&](auto ii) {
                constexpr int ic = decltype(ii)::value;
                if (ic != i) return;
                Unroll<0, TN>::run([&](auto jj) {
                    constexpr int j = decltype(jj)::value;
                    Unroll<0, NG>::run([&](auto gg) {
                        constexpr int g = decltype(gg)::value;
                        *reinterpret_cast<f32x4 *>(stage + acc_row<MF>(lane) * SROW + j * MF +
                                                   acc_col<MF>(lane, g)) =
                            acc_group<AGPR>(acc[ic][j], g);
                    });
                });
            });
            // (LDS operations of one wave complete in order; this only keeps
            // the compiler from moving the reads above the writes)
            __builtin_amdgcn_wave_barrier();
            if constexpr (IT != IT_I8) {
                if (p.splits == 1 && p.cd_vec && (p.C || p.epi)) {
                    if (p.out_dtype == DT_F32) linear(std::integral_constant<int, DT_F32>{}, i);
                    else if (p.out_dtype == DT_F16) linear(std::integral_constant<int, DT_F16>{}, i);
                    else linear(std::integral_constant<int, DT_BF16>{}, i);
                }
            }
            for (int rr = lane / LPR; rr < MF; rr += RPP) {
                const f32x4 v = *reinterpret_cast<const f32x4 *>(stage + rr * SROW + c4);
                const int gi = row0 + i * MF + rr;
                // a group inside M x N of an edge tile still takes the vector
                // finish (C, D and bias alignment are tile-independent)
                const bool gfull = gfull_at(gi);
                if (p.splits > 1) {
                    finish4<-1, false, false>(p, gi, gj, v);
                } else if constexpr (IT == IT_I8) {  // int32 out, plain epilogue only
                    if (gfull) finish4<DT_I32, true, false>(p, gi, gj, v);
                    else finish4<DT_I32, false, false>(p, gi, gj, v);
                } else if (p.epi) {
                    if (gfull) {
                        if (p.out_dtype == DT_F32) finish4<DT_F32, true, true, true>(p, gi, gj, v);
                        else if (p.out_dtype == DT_F16) finish4<DT_F16, true, true, true>(p, gi, gj, v);
                        else finish4<DT_BF16, true, true, true>(p, gi, gj, v);
                    } else {
                        if (p.out_dtype == DT_F32) finish4<DT_F32, false, true>(p, gi, gj, v);
                        else if (p.out_dtype == DT_F16) finish4<DT_F16, false, true>(p, gi, gj, v);
                        else finish4<DT_BF16, false, true>(p, gi, gj, v);
                    }
                } else if (gfull) {
                    if (p.out_dtype == DT_F32) finish4<DT_F32, true, false, true>(p, gi, gj, v);
                    else if (p.out_dtype == DT_F16) finish4<DT_F16, true, false, true>(p, gi, gj, v);
                    else finish4<DT_BF16, true, false, true>(p, gi, gj, v);
                } else {
                    if (p.out_dtype == DT_F32) finish4<DT_F32, false, false>(p, gi, gj, v);
                    else if (p.out_dtype == DT_F16) finish4<DT_F16, false, false>(p, gi, gj, v);
                    else finish4<DT_BF16, false, false>(p, gi, gj, v);
                }
            }
            __builtin_amdgcn_wave_barrier();
        }
    }
}

// ------------------------------------------------------------------ kernel
// VEC selects the vector (aligned) or the element-wise (unaligned) loads and
// RAGGED whether the vector loads mask k >= kend; each combination is its own
// kernel, with a single K loop to allocate registers for.
template <class CF, int IT, bool A_KC, bool B_KC, bool VEC, bool RAGGED>
__global__ void __launch_bounds__(CF::THREADS) gemm_mfma_kernel(Params p) {
    constexpr int BM = CF::BM, BN = CF::BN, CH = CF::CH;
    constexpr int MF = CF::MF, TM = CF::TM, TN = CF::TN;
    using Acc = typename AccT<MF>::type;

    __shared__ u32x4 smem[2 * (BM + BN) * CH];
    u32x4 *const sA = smem;                 // [2][BM*CH]
    u32x4 *const sB = smem + 2 * BM * CH;   // [2][BN*CH]

    const int tid = threadIdx.x;
    int tile_m, tile_n;
    map_tile(p, blockIdx.x, tile_m, tile_n);
    const int m0 = tile_m * BM, n0 = tile_n * BN;

    const int kbeg = blockIdx.z * p.k_per_split;
    const int kend = min(p.K, kbeg + p.k_per_split);

    Acc acc[TM][TN];
    Unroll<0, TM>::run([&](auto ii) {
        Unroll<0, TN>::run([&](auto jj) {
            acc[decltype(ii)::value][decltype(jj)::value] = Acc{};
        });
    });

    k_loop<CF, IT, A_KC, B_KC, VEC, RAGGED>(p, m0, n0, kbeg, kend, acc, sA, sB, tid);
    tile_epilogue<CF, IT, VEC, (int)sizeof(smem), false, !RAGGED>(p, acc, m0, n0, smem, tid);
}

// Large tiles on the LDS-DMA K loop (operands with 16-byte aligned rows, in
// every layout; the host sends no others).
template <class CF, int IT, bool A_KC, bool B_KC, bool RAGGED>
__global__ void __launch_bounds__(CF::THREADS) gemm_dma_kernel(Params p) {
    constexpr int BM = CF::BM, BN = CF::BN, BK = CF::BK;
    constexpr int MF = CF::MF, TM = CF::TM, TN = CF::TN;
    using Acc = typename AccT<MF>::type;

    // two stages of A and B, then the 1 KiB sink of the K loop's idle DMA
    __shared__ u32x4 smem[2 * (BM + BN) * BK * CF::ES / 16 + 64];
    const int tid = threadIdx.x;
    int tile_m, tile_n;
    map_tile(p, blockIdx.x, tile_m, tile_n);
    const int m0 = tile_m * BM, n0 = tile_n * BN;
    const int kbeg = blockIdx.z * p.k_per_split;
    const int kend = min(p.K, kbeg + p.k_per_split);

    Acc acc[TM][TN];
    Unroll<0, TM>::run([&](auto ii) {
        Unroll<0, TN>::run([&](auto jj) {
            acc[decltype(ii)::value][decltype(jj)::value] = Acc{};
        });
    });
    dma_k_loop<CF, IT, A_KC, B_KC, RAGGED>(p, m0, n0, kbeg, kend, acc,
                                           reinterpret_cast<char *>(smem), tid);
    tile_epilogue<CF, IT, true, 2 * (BM + BN) * BK * CF::ES, true>(p, acc, m0, n0, smem, tid);
    wait_vmcnt<0>();  // the sink's loads land before the workgroup's LDS is released
}

}  // namespace libgemm
