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

namespace libgemm {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

enum { DT_F32 = 0, DT_F16 = 1, DT_BF16 = 2 };

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
    int tiles_m, tiles_n;
    int splits;      // K slices (blockIdx.z); 1 = no split
    int k_per_split; // multiple of BK
};

// Block-tile configuration.  MF = 32 selects the 32x32x16 MFMA, 16 the
// 16x16x32 one.  Waves form a WAVES_M x WAVES_N grid over the block tile.
template <int BM_, int BN_, int BK_, int WAVES_M_, int WAVES_N_, int MF_, int GROUP_M_>
struct TileCfg {
    static constexpr int BM = BM_, BN = BN_, BK = BK_;
    static constexpr int WAVES_M = WAVES_M_, WAVES_N = WAVES_N_;
    static constexpr int THREADS = 64 * WAVES_M * WAVES_N;
    static constexpr int MF = MF_;
    static constexpr int KSTEP = (MF == 32) ? 16 : 32;  // k consumed by one MFMA
    static constexpr int WTM = BM / WAVES_M, WTN = BN / WAVES_N;
    static constexpr int TM = WTM / MF, TN = WTN / MF;
    static constexpr int CH = BK / 8;  // 16-byte chunks per LDS row
    static constexpr int GROUP_M = GROUP_M_;
    static_assert(MF == 32 || MF == 16, "MFMA shape");
    static_assert(BK % 64 == 0, "the LDS swizzle assumes rows of >= 128 bytes");
    static_assert(WTM % MF == 0 && WTN % MF == 0, "wave tile");
    static_assert(BM % 8 == 0 && BN % 8 == 0, "row groups of 8");
};

// ---------------------------------------------------------------- LDS layout
// Row r of an operand tile holds BK k-values (CH chunks of 8).  Chunk c is
// stored at position c ^ swz(r).  Eight consecutive rows read at one chunk,
// and eight rows 8 apart written at one chunk, land in eight different
// 16-byte bank groups.
__device__ __forceinline__ int swz(int r) { return (r ^ (r >> 3)) & 7; }

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
// Each loader fetches one ROWS x BK tile into registers (load_*) and writes
// it to LDS K-contiguous (store).

template <int ROWS, int BK, int THREADS>
struct LoaderKC {
    static constexpr int CH = BK / 8;
    static constexpr int TOTAL = ROWS * CH;  // 16-byte chunks in the tile
    static constexpr bool PARTIAL = TOTAL < THREADS;
    static constexpr int PER = PARTIAL ? 1 : TOTAL / THREADS;
    static_assert(PARTIAL || TOTAL % THREADS == 0, "tile/threads");
    u32x4 v[PER];

    __device__ __forceinline__ void load_fast(const uint16_t *X, int64_t ld, int r0, int k0,
                                              int tid) {
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int q = i * THREADS + tid;
            if (PARTIAL && q >= TOTAL) break;
            const int r = q / CH, c = q % CH;
            v[i] = *reinterpret_cast<const u32x4 *>(X + (int64_t)(r0 + r) * ld + (k0 + c * 8));
        }
    }

    __device__ __forceinline__ void load_checked(const uint16_t *X, int64_t ld, int r0, int k0,
                                                 int R, int Kend, int vec_ok, int tid) {
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int q = i * THREADS + tid;
            if (PARTIAL && q >= TOTAL) break;
            const int r = q / CH, c = q % CH;
            const int gr = r0 + r, gk = k0 + c * 8;
            if (gr < R && gk + 8 <= Kend && vec_ok) {
                v[i] = *reinterpret_cast<const u32x4 *>(X + (int64_t)gr * ld + gk);
            } else {
                uint32_t h[8];
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    h[e] = (gr < R && gk + e < Kend) ? (uint32_t)X[(int64_t)gr * ld + gk + e] : 0u;
                v[i] = u32x4{h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16),
                             h[6] | (h[7] << 16)};
            }
        }
    }

    __device__ __forceinline__ void store(u32x4 *lds, int tid) const {
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int q = i * THREADS + tid;
            if (PARTIAL && q >= TOTAL) break;
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
    static_assert(PARTIAL || TOTAL % THREADS == 0, "tile/threads");
    static_assert(KB == 1 || KB == 2 || KB == 4 || KB == 8, "k-depth");
    static_assert(PERT % KB == 0, "blocks");
    static_assert(BK % KB == 0, "k groups");
    u32x4 v[NBLK][KB];  // v[j][kk]: 8 consecutive r at k = kg*KB + kk

    // block b -> (kg, rb): rb fastest, so adjacent lanes read adjacent 16 B
    __device__ __forceinline__ void load_fast(const uint16_t *X, int64_t ld, int r0, int k0,
                                              int tid) {
#pragma unroll
        for (int j = 0; j < NBLK; ++j) {
            const int b = j * THREADS + tid;
            if (PARTIAL && b >= NBLOCKS) break;
            const int rb = b % RCH, kg = b / RCH;
            const uint16_t *src = X + (int64_t)(k0 + kg * KB) * ld + (r0 + rb * 8);
#pragma unroll
            for (int kk = 0; kk < KB; ++kk)
                v[j][kk] = *reinterpret_cast<const u32x4 *>(src + (int64_t)kk * ld);
        }
    }

    __device__ __forceinline__ void load_checked(const uint16_t *X, int64_t ld, int r0, int k0,
                                                 int R, int Kend, int vec_ok, int tid) {
#pragma unroll
        for (int j = 0; j < NBLK; ++j) {
            const int b = j * THREADS + tid;
            if (PARTIAL && b >= NBLOCKS) break;
            const int rb = b % RCH, kg = b / RCH;
            const int gr = r0 + rb * 8;
#pragma unroll
            for (int kk = 0; kk < KB; ++kk) {
                const int gk = k0 + kg * KB + kk;
                const uint16_t *src = X + (int64_t)gk * ld + gr;
                if (gk < Kend && gr + 8 <= R && vec_ok) {
                    v[j][kk] = *reinterpret_cast<const u32x4 *>(src);
                } else {
                    uint32_t h[8];
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        h[e] = (gk < Kend && gr + e < R) ? (uint32_t)src[e] : 0u;
                    v[j][kk] = u32x4{h[0] | (h[1] << 16), h[2] | (h[3] << 16),
                                     h[4] | (h[5] << 16), h[6] | (h[7] << 16)};
                }
            }
        }
    }

    // Transpose each KB x 8 block in registers: LDS row (rb*8 + e) receives
    // the KB k-values of column e, at k offset kg*KB.
    __device__ __forceinline__ void store(u32x4 *lds, int tid) const {
        constexpr int CH = BK / 8;
#pragma unroll
        for (int j = 0; j < NBLK; ++j) {
            const int b = j * THREADS + tid;
            if (PARTIAL && b >= NBLOCKS) break;
            const int rb = b % RCH, kg = b / RCH;
            const int kofs = kg * KB;
            const int c = kofs / 8, sub = kofs % 8;  // chunk and element offset
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int r = rb * 8 + e;
                u32x4 *dst = lds + r * CH + (c ^ swz(r));
                if constexpr (KB == 8) {
                    u32x4 w;
#pragma unroll
                    for (int p = 0; p < 4; ++p)
                        w[p] = half_of(v[j][2 * p], e) | (half_of(v[j][2 * p + 1], e) << 16);
                    *dst = w;
                } else if constexpr (KB == 4) {
                    u32x2 w;
                    w[0] = half_of(v[j][0], e) | (half_of(v[j][1], e) << 16);
                    w[1] = half_of(v[j][2], e) | (half_of(v[j][3], e) << 16);
                    reinterpret_cast<u32x2 *>(dst)[sub / 4] = w;
                } else if constexpr (KB == 2) {
                    reinterpret_cast<uint32_t *>(dst)[sub / 2] =
                        half_of(v[j][0], e) | (half_of(v[j][1], e) << 16);
                } else {
                    reinterpret_cast<uint16_t *>(dst)[sub] = (uint16_t)half_of(v[j][0], e);
                }
            }
        }
    }
};

// ------------------------------------------------------------------- MFMA
template <bool BF>
__device__ __forceinline__ f32x16 mfma32(const u32x4 &a, const u32x4 &b, const f32x16 &c) {
    if constexpr (BF)
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                      __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

template <bool BF>
__device__ __forceinline__ f32x4 mfma16(const u32x4 &a, const u32x4 &b, const f32x4 &c) {
    if constexpr (BF)
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                      __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

template <int MF> struct AccT;
template <> struct AccT<32> { typedef f32x16 type; static constexpr int N = 16; };
template <> struct AccT<16> { typedef f32x4 type; static constexpr int N = 4; };

// Position of accumulator register r of `lane` inside an MF x MF tile.
// 32x32: column lane%32, row 8*(r/4) + 4*(lane/32) + r%4.
// 16x16: column lane%16, row 4*(lane/16) + r.
template <int MF>
__device__ __forceinline__ int acc_row(int lane, int r) {
    if constexpr (MF == 32)
        return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
    else
        return 4 * (lane >> 4) + r;
}
template <int MF>
__device__ __forceinline__ int acc_col(int lane) { return lane & (MF - 1); }

// ---------------------------------------------------------------- epilogue
__device__ __forceinline__ float load_c(const Params &p, int64_t i, int64_t j) {
    const int64_t off = i * p.ldc + j;
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

// v = acc (+ C), rounded once to the output dtype OUT, then satf, stored at
// D(i,j).  OUT is a template argument so the hot epilogue has no dtype branch.
template <int OUT>
__device__ __forceinline__ void finish_store_t(const Params &p, int64_t i, int64_t j, float v) {
    if (p.C) v += load_c(p, i, j);
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

// ------------------------------------------------------------ tile mapping
// Workgroups are handed to the 8 XCDs round-robin (workgroup w runs on XCD
// w % 8).  Renumber them so each XCD receives a contiguous range of tiles,
// then walk tiles in groups of GROUP_M tile-rows, so the tiles that share
// A row-panels and B column-panels run on the same XCD's L2.
template <int GROUP_M>
__device__ __forceinline__ void map_tile(const Params &p, int w, int &tm, int &tn) {
    const int T = p.tiles_m * p.tiles_n;
    const int xcd = w & 7, local = w >> 3;
    const int per = T >> 3, rem = T & 7;
    const int t = xcd * per + (xcd < rem ? xcd : rem) + local;
    const int in_group = GROUP_M * p.tiles_n;
    const int g = t / in_group;
    const int first_m = g * GROUP_M;
    const int gsize = (p.tiles_m - first_m) < GROUP_M ? (p.tiles_m - first_m) : GROUP_M;
    const int t_in = t - g * in_group;
    tm = first_m + t_in % gsize;
    tn = t_in / gsize;
}

// ------------------------------------------------------------------ kernel
template <class CF, bool BF, bool A_KC, bool B_KC>
__global__ void __launch_bounds__(CF::THREADS) gemm_mfma_kernel(Params p) {
    constexpr int BM = CF::BM, BN = CF::BN, BK = CF::BK, CH = CF::CH;
    constexpr int MF = CF::MF, TM = CF::TM, TN = CF::TN, THREADS = CF::THREADS;
    using LA = typename std::conditional<A_KC, LoaderKC<BM, BK, THREADS>,
                                         LoaderRC<BM, BK, THREADS>>::type;
    using LB = typename std::conditional<B_KC, LoaderKC<BN, BK, THREADS>,
                                         LoaderRC<BN, BK, THREADS>>::type;
    using Acc = typename AccT<MF>::type;

    __shared__ u32x4 smem[2 * (BM + BN) * CH];
    u32x4 *const sA = smem;                 // [2][BM*CH]
    u32x4 *const sB = smem + 2 * BM * CH;   // [2][BN*CH]

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave / CF::WAVES_N, wn = wave % CF::WAVES_N;

    int tile_m, tile_n;
    map_tile<CF::GROUP_M>(p, blockIdx.x, tile_m, tile_n);
    const int m0 = tile_m * BM, n0 = tile_n * BN;

    const int kbeg = blockIdx.z * p.k_per_split;
    const int kend = min(p.K, kbeg + p.k_per_split);
    const int nk = kend > kbeg ? (kend - kbeg + BK - 1) / BK : 0;
    const bool interior = p.vec_ok && (m0 + BM <= p.M) && (n0 + BN <= p.N);

    LA la;
    LB lb;
    Acc acc[TM][TN];
    Unroll<0, TM>::run([&](auto ii) {
        Unroll<0, TN>::run([&](auto jj) {
            acc[decltype(ii)::value][decltype(jj)::value] = Acc{};
        });
    });

    auto load_tiles = [&](int kt) {
        const int k0 = kbeg + kt * BK;
        if (interior && k0 + BK <= kend) {
            la.load_fast(p.A, p.lda, m0, k0, tid);
            lb.load_fast(p.B, p.ldb, n0, k0, tid);
        } else {
            la.load_checked(p.A, p.lda, m0, k0, p.M, kend, p.vec_ok, tid);
            lb.load_checked(p.B, p.ldb, n0, k0, p.N, kend, p.vec_ok, tid);
        }
    };

    if (nk > 0) {
        load_tiles(0);
        la.store(sA, tid);
        lb.store(sB, tid);
    }
    __syncthreads();

    for (int kt = 0; kt < nk; ++kt) {
        const int cur = kt & 1;
        if (kt + 1 < nk) load_tiles(kt + 1);  // in flight during the MFMAs below

        const u32x4 *a_s = sA + cur * BM * CH;
        const u32x4 *b_s = sB + cur * BN * CH;
#pragma unroll
        for (int ks = 0; ks < BK / CF::KSTEP; ++ks) {
            u32x4 af[TM], bf[TN];
            const int chunk = ks * (CF::KSTEP / 8) + lane / MF;
#pragma unroll
            for (int i = 0; i < TM; ++i) {
                const int r = wm * CF::WTM + i * MF + (lane & (MF - 1));
                af[i] = a_s[r * CH + (chunk ^ swz(r))];
            }
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                const int r = wn * CF::WTN + j * MF + (lane & (MF - 1));
                bf[j] = b_s[r * CH + (chunk ^ swz(r))];
            }
            Unroll<0, TM>::run([&](auto ii) {
                Unroll<0, TN>::run([&](auto jj) {
                    constexpr int i = decltype(ii)::value, j = decltype(jj)::value;
                    if constexpr (MF == 32)
                        acc[i][j] = mfma32<BF>(af[i], bf[j], acc[i][j]);
                    else
                        acc[i][j] = mfma16<BF>(af[i], bf[j], acc[i][j]);
                });
            });
        }

        if (kt + 1 < nk) {
            la.store(sA + (cur ^ 1) * BM * CH, tid);
            lb.store(sB + (cur ^ 1) * BN * CH, tid);
        }
        __syncthreads();
    }

    // Epilogue: split-K slices store raw fp32 partial sums (OUT = -1);
    // otherwise C add, convert, satf and store.  Interior tiles skip the
    // bounds checks.
    const bool full_tile = (m0 + BM <= p.M) && (n0 + BN <= p.N);
    auto epilogue = [&](auto out_tag, auto check_tag) {
        constexpr int OUT = decltype(out_tag)::value;
        constexpr bool CHECK = decltype(check_tag)::value;
        Unroll<0, TM>::run([&](auto ii) {
            Unroll<0, TN>::run([&](auto jj) {
                Unroll<0, AccT<MF>::N>::run([&](auto rr) {
                    constexpr int i = decltype(ii)::value, j = decltype(jj)::value;
                    constexpr int r = decltype(rr)::value;
                    const int gi = m0 + wm * CF::WTM + i * MF + acc_row<MF>(lane, r);
                    const int gj = n0 + wn * CF::WTN + j * MF + acc_col<MF>(lane);
                    if (!CHECK || (gi < p.M && gj < p.N)) {
                        if constexpr (OUT < 0)
                            p.ws[((int64_t)blockIdx.z * p.M + gi) * p.N + gj] = acc[i][j][r];
                        else
                            finish_store_t<OUT>(p, gi, gj, acc[i][j][r]);
                    }
                });
            });
        });
    };
    using IC_T = std::integral_constant<bool, true>;
    using IC_F = std::integral_constant<bool, false>;
    if (p.splits > 1) {
        epilogue(std::integral_constant<int, -1>{}, IC_T{});
    } else if (p.out_dtype == DT_F32) {
        if (full_tile) epilogue(std::integral_constant<int, DT_F32>{}, IC_F{});
        else epilogue(std::integral_constant<int, DT_F32>{}, IC_T{});
    } else if (p.out_dtype == DT_F16) {
        if (full_tile) epilogue(std::integral_constant<int, DT_F16>{}, IC_F{});
        else epilogue(std::integral_constant<int, DT_F16>{}, IC_T{});
    } else {
        if (full_tile) epilogue(std::integral_constant<int, DT_BF16>{}, IC_F{});
        else epilogue(std::integral_constant<int, DT_BF16>{}, IC_T{});
    }
}

}  // namespace libgemm
