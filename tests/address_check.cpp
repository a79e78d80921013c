// Host check of the operand-load address arithmetic (gemm_address.hpp), as
// the kernels' loaders compose it: for every tile, thread, chunk and K-tile
// of a problem, the 16-byte chunk read
//   - lies inside the operand's extent rounded up to 16 bytes, and
//   - holds at least one element of the matrix (row < R, k < K),
// and every chunk whose values are used (row < R, k < kend) is the chunk the
// definition names.  Built with a plain C++ compiler by
// tests/test_address_cpu.py; prints one line per failure and exits nonzero.
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include <initializer_list>
#include <vector>

#include "gemm_address.hpp"

using namespace libgemm;

static long g_fail = 0, g_checked = 0;

static void fail(const char *what, long a, long b, long c, long d) {
    if (g_fail < 20) printf("FAIL %s: %ld %ld %ld %ld\n", what, a, b, c, d);
    ++g_fail;
}

// K-contiguous loader: ROWS x BK tile as CH = BK*ES/16 chunks per row, THREADS
// threads, chunk q = i*THREADS + tid (or tid % TOTAL for partial tiles).
static void check_kc(int ROWS, int BK, int THREADS, int ES, int R, int K, int64_t ld, int kps) {
    const int CH = BK * ES / 16, EPC = 16 / ES;
    const int TOTAL = ROWS * CH;
    const bool partial = TOTAL < THREADS;
    const int PER = partial ? 1 : TOTAL / THREADS;
    const int64_t range = operand_range(R, K, ld, ES);
    const int splits = (K + kps - 1) / kps;
    const bool ragged = (K % BK) != 0 || (kps % BK) != 0;
    for (int r0 = 0; r0 < R; r0 += ROWS)
        for (int z = 0; z < splits; ++z) {
            const int kbeg = z * kps, kend = K < kbeg + kps ? K : kbeg + kps;
            for (int k0 = kbeg; k0 < kend; k0 += BK)
                for (int tid = 0; tid < THREADS; ++tid)
                    for (int i = 0; i < PER; ++i) {
                        const int q = partial ? tid % TOTAL : i * THREADS + tid;
                        const int kc = (q % CH) * EPC;
                        const int r = r0 + q / CH;
                        // what the loader computes: voff at k0 = 0, then the
                        // k position (scalar offset, or clamped in RAGGED)
                        const int64_t voff = kc_chunk_offset(r, kc, R, 1, ld, ES, false);
                        const int64_t off = ragged ? voff - kc * ES + kc_k_offset(k0 + kc, kend, ES)
                                                   : voff + (int64_t)k0 * ES;
                        ++g_checked;
                        if (off < 0 || off % 16 != 0 || off + 16 > range)
                            fail("kc out of range", off, range, r, k0 + kc);
                        const int rr = r < R ? r : R - 1;
                        const int64_t in_row = off / ES - (int64_t)rr * ld;
                        if (in_row < 0 || in_row >= K) fail("kc chunk holds no element", off, rr, in_row, K);
                        if (r < R && k0 + kc < kend && off != ((int64_t)r * ld + k0 + kc) * ES)
                            fail("kc wrong chunk", off, r, k0 + kc, 0);
                    }
        }
}

// R-contiguous loader (16-bit): 8 consecutive rows r at one k per chunk.
static void check_rc(int ROWS, int BK, int THREADS, int R, int K, int64_t ld, int kps) {
    const int RCH = ROWS / 8;
    const int TOTAL = RCH * BK;
    const bool partial = TOTAL < THREADS;
    const int PERT = partial ? 1 : TOTAL / THREADS;
    const int KB = PERT < 8 ? PERT : 8;
    const int NBLK = PERT / KB, NBLOCKS = TOTAL / KB;
    // the loader's block -> (rb, kg) map: adjacent lanes pair up on one rb
    const bool pairs = NBLOCKS % (2 * RCH) == 0 && (partial || THREADS % (2 * RCH) == 0);
    auto rb_of = [&](int b) { return pairs ? (b >> 1) % RCH : b % RCH; };
    auto kg_of = [&](int b) { return pairs ? (b & 1) + 2 * (b / (2 * RCH)) : b / RCH; };
    {   // a bijection onto the tile's blocks, and rb the same for all of a thread's blocks
        char *seen = (char *)calloc(NBLOCKS, 1);
        for (int tid = 0; tid < THREADS; ++tid)
            for (int j = 0; j < NBLK; ++j) {
                const int b = partial ? tid % NBLOCKS : j * THREADS + tid;
                const int b0 = partial ? tid % NBLOCKS : tid;
                if (rb_of(b) != rb_of(b0)) fail("rc rb differs across blocks", tid, j, ROWS, BK);
                const int id = kg_of(b) * RCH + rb_of(b);
                if (id < 0 || id >= NBLOCKS) fail("rc block out of range", tid, j, id, NBLOCKS);
                else seen[id] = 1;
            }
        for (int id = 0; id < NBLOCKS; ++id)
            if (!seen[id]) fail("rc block not covered", id, ROWS, BK, THREADS);
        free(seen);
    }
    const int64_t range = operand_range(K, R, ld, 2);
    const int splits = (K + kps - 1) / kps;
    const bool ragged = (K % BK) != 0 || (kps % BK) != 0;
    for (int r0 = 0; r0 < R; r0 += ROWS)
        for (int z = 0; z < splits; ++z) {
            const int kbeg = z * kps, kend = K < kbeg + kps ? K : kbeg + kps;
            for (int k0 = kbeg; k0 < kend; k0 += BK)
                for (int tid = 0; tid < THREADS; ++tid)
                    for (int j = 0; j < NBLK; ++j)
                        for (int kk = 0; kk < KB; ++kk) {
                            const int b = partial ? tid % NBLOCKS : j * THREADS + tid;
                            const int rb = rb_of(b), kg = kg_of(b);
                            const int col = r0 + rb * 8;
                            const int64_t voff = rc_chunk_offset(col, 0, R, 1, 0, false);
                            const int k = k0 + kg * KB + kk;
                            const int64_t off = ragged ? voff + (int64_t)imin(k, kend - 1) * ld * 2
                                                       : voff + (int64_t)(kg * KB + kk) * ld * 2 +
                                                             (int64_t)k0 * ld * 2;
                            ++g_checked;
                            if (off < 0 || off % 16 != 0 || off + 16 > range)
                                fail("rc out of range", off, range, col, k);
                            const int64_t row = off / (ld * 2), c0 = (off % (ld * 2)) / 2;
                            if (row >= K || c0 >= R) fail("rc chunk holds no element", off, row, c0, R);
                            if (col < R && k < kend && off != ((int64_t)k * ld + col) * 2)
                                fail("rc wrong chunk", off, col, k, 0);
                        }
        }
}

// R-contiguous loader (8-bit): blocks of 4 rows x 16 k-rows, one dword per
// k-row, then the in-register transpose (rc8_gather) into the 4 rows'
// K-contiguous chunks.  Checks the dword reads like check_rc, the block map,
// and that the transposed chunk of row r at k-group kg holds X(r, 16kg..+15).
static uint8_t code8(int64_t off) { return (uint8_t)((off * 2654435761u) >> 13); }

static void check_rc8(int ROWS, int BK, int THREADS, int R, int K, int64_t ld, int kps) {
    const int RG = ROWS / 4, KG = BK / 16;
    const int TOTAL = RG * KG;
    const bool partial = TOTAL < THREADS;
    const int NBLK = partial ? 1 : TOTAL / THREADS;
    {   // every block covered; the row group the same for all of a thread's blocks
        char *seen = (char *)calloc(TOTAL, 1);
        for (int tid = 0; tid < THREADS; ++tid)
            for (int j = 0; j < NBLK; ++j) {
                const int b = partial ? tid % TOTAL : j * THREADS + tid;
                const int b0 = partial ? tid % TOTAL : tid;
                if (b % RG != b0 % RG) fail("rc8 row group differs across blocks", tid, j, ROWS, BK);
                if (b < 0 || b >= TOTAL) fail("rc8 block out of range", tid, j, b, TOTAL);
                else seen[b] = 1;
            }
        for (int id = 0; id < TOTAL; ++id)
            if (!seen[id]) fail("rc8 block not covered", id, ROWS, BK, THREADS);
        free(seen);
    }
    const int64_t range = operand_range(K, R, ld, 1);
    const int splits = (K + kps - 1) / kps;
    const bool ragged = (K % BK) != 0 || (kps % BK) != 0;
    for (int r0 = 0; r0 < R; r0 += ROWS)
        for (int z = 0; z < splits; ++z) {
            const int kbeg = z * kps, kend = K < kbeg + kps ? K : kbeg + kps;
            for (int k0 = kbeg; k0 < kend; k0 += BK)
                for (int tid = 0; tid < THREADS; ++tid)
                    for (int j = 0; j < NBLK; ++j) {
                        const int b = partial ? tid % TOTAL : j * THREADS + tid;
                        const int rg = b % RG, kg = b / RG;
                        const int col = r0 + rg * 4;
                        const int64_t voff = rc8_dword_offset(col, 0, R, 1, ld, false);
                        uint32_t v[16];
                        for (int kk = 0; kk < 16; ++kk) {
                            const int k = k0 + kg * 16 + kk;
                            const int64_t off = ragged ? voff + (int64_t)imin(k, kend - 1) * ld
                                                       : voff + (int64_t)(kg * 16 + kk) * ld +
                                                             (int64_t)k0 * ld;
                            ++g_checked;
                            if (off < 0 || off % 4 != 0 || off + 4 > range)
                                fail("rc8 out of range", off, range, col, k);
                            const int64_t row = off / ld, c0 = off % ld;
                            if (row >= K || c0 >= R) fail("rc8 dword holds no element", off, row, c0, R);
                            if (col < R && k < kend && off != (int64_t)k * ld + col)
                                fail("rc8 wrong dword", off, col, k, 0);
                            // the dword's bytes, masked to zero for k >= kend
                            v[kk] = 0;
                            for (int e = 0; e < 4; ++e)
                                v[kk] |= (uint32_t)(k < kend ? code8(off + e) : 0) << (8 * e);
                        }
                        // the transposed chunk of each of the 4 rows
                        for (int e = 0; e < 4; ++e) {
                            const int r = col + e;
                            if (r >= R) continue;
                            for (int d = 0; d < 4; ++d) {
                                const uint32_t w = rc8_gather(v[4 * d], v[4 * d + 1], v[4 * d + 2],
                                                              v[4 * d + 3], e);
                                for (int q = 0; q < 4; ++q) {
                                    const int k = k0 + kg * 16 + 4 * d + q;
                                    const uint8_t want = k < kend ? code8((int64_t)k * ld + r) : 0;
                                    if (((w >> (8 * q)) & 0xffu) != want)
                                        fail("rc8 transposed byte", r, k, (w >> (8 * q)) & 0xffu, want);
                                }
                            }
                        }
                    }
        }
}

// --------------------------------------------------------- LDS-DMA path
// One operand tile of ROWS x BK 16-bit values through the DMA kernel's data
// path, simulated: the value of X(r, k) is a unique code; the DMA mapping
// (dma_kc_source / dma_rc_source) fills an LDS image chunk by chunk, then
// every fragment read of every step is performed as the kernel does it --
// ds_read_b128 at the KC offset, or two ds_read_b64_tr_b16 at
// tr_read_offset with the instruction's lane exchange -- and each lane must
// hold X(rb + lane % MF, k0 + 8 * (lane / MF) + e), e = 0..7, the MFMA's
// operand layout.
static uint16_t code(int r, int k) { return (uint16_t)(((r & 0x3ff) << 6) ^ (k * 40503u)); }

// perm: K-contiguous 16x16 reads in the kc_group16 order (both operands
// K-contiguous), lane group g then holding k-group kc_group16(g)
static void check_dma_tile(int ROWS, int BK, int MF, bool KC, int nwaves, bool perm = false) {
    const int bytes = ROWS * BK * 2, chunks = bytes / 16;
    const int ni = bytes / 1024 / nwaves;
    if (bytes % (1024 * nwaves)) { fail("dma blocks", ROWS, BK, nwaves, 0); return; }
    uint16_t *lds = (uint16_t *)calloc(chunks * 8, 2);
    int *filled = (int *)calloc(chunks, sizeof(int));
    for (int w = 0; w < nwaves; ++w)
        for (int i = 0; i < ni; ++i)
            for (int l = 0; l < 64; ++l) {
                const int q = (w * ni + i) * 64 + l;   // the LDS chunk lane l fills
                int a, c;
                if (KC) dma_kc_source(q, BK / 8, a, c); else dma_rc_source(q, ROWS / 8, MF, a, c);
                for (int e = 0; e < 8; ++e)   // KC: row a, k = 8c+e; RC: k-row a, row 8c+e
                    lds[q * 8 + e] = KC ? code(a, 8 * c + e) : code(8 * c + e, a);
                filled[q]++;
            }
    for (int q = 0; q < chunks; ++q)
        if (filled[q] != 1) fail("dma chunk filled times", q, filled[q], ROWS, KC);
    const int kstep = MF == 32 ? 16 : 32;
    for (int ks = 0; ks < BK / kstep; ++ks)
        for (int rb = 0; rb < ROWS; rb += MF) {
            uint16_t got[64][8];
            if (KC) {
                const int kch = kstep * 2 / 16;
                for (int lane = 0; lane < 64; ++lane) {
                    const int r = rb + lane % MF;
                    const int lg = perm ? kc_group16(lane / MF) : lane / MF;
                    const uint32_t off = (uint32_t)(r * (BK / 8) + (lg ^ swz_kc(r))) * 16u;
                    const uint32_t a = off ^ (uint32_t)(ks * kch * 16);
                    for (int e = 0; e < 8; ++e) got[lane][e] = lds[a / 2 + e];
                }
            } else {
                for (int h = 0; h < 2; ++h) {
                    uint16_t in[64][4];
                    for (int L = 0; L < 64; ++L) {
                        const int off = tr_read_offset(L, MF, ks, h, rb, ROWS * 2);
                        if (off % 8 || off < 0 || off + 8 > bytes) fail("tr offset", off, L, ks, h);
                        for (int e = 0; e < 4; ++e) in[L][e] = lds[off / 2 + e];
                    }
                    // the instruction's exchange: lane j element f <- lane
                    // 16*(j/16) + 4f + (j%16)/4, element j%4
                    for (int j = 0; j < 64; ++j)
                        for (int f = 0; f < 4; ++f)
                            got[j][4 * h + f] = in[16 * (j / 16) + 4 * f + (j % 16) / 4][j % 4];
                }
            }
            for (int lane = 0; lane < 64; ++lane)
                for (int e = 0; e < 8; ++e) {
                    const int lg = perm ? kc_group16(lane / MF) : lane / MF;
                    const int r = rb + lane % MF, k = ks * kstep + 8 * lg + e;
                    ++g_checked;
                    if (got[lane][e] != code(r, k)) fail("fragment value", lane, e, r, k);
                }
        }
    free(lds);
    free(filled);
}

// The 8-bit DMA tile (ROWS x BK bytes, fc 16-byte chunks per lane and MFMA
// operand, the 32x32 MFMA): every byte is tracked by the element it holds.
// The DMA placement fills each LDS chunk once; the fragment reads (KC: fc
// 16-byte reads; RC: 2*fc transposed reads with the exchange probed on the
// GPU) must give lane j the bytes X(rb + j % 32, k) for
// k = ks*kstep + 16*fc*(j / 32) + 16c + e, e = 0..15, chunk c < fc; and each
// half-wave of a transposed read must touch 64 distinct 4-byte banks.
static void check_dma_tile8(int ROWS, int BK, int fc, bool KC, int nwaves) {
    const int bytes = ROWS * BK, chunks = bytes / 16;
    const int ni = bytes / 1024 / nwaves;
    const int kstep = 32 * fc;
    if (bytes % (1024 * nwaves)) { fail("dma8 blocks", ROWS, BK, nwaves, 0); return; }
    std::vector<int> lds((size_t)bytes, -1), filled((size_t)chunks, 0);
    auto id = [](int r, int k) { return r * 4096 + k; };
    for (int w = 0; w < nwaves; ++w)
        for (int i = 0; i < ni; ++i)
            for (int l = 0; l < 64; ++l) {
                const int q = (w * ni + i) * 64 + l;
                int a, c;
                if (KC) dma_kc_source(q, BK / 16, a, c); else dma_rc8_source(q, ROWS / 16, a, c);
                for (int e = 0; e < 16; ++e)   // KC: row a, k = 16c+e; RC: k-row a, row 16c+e
                    lds[(size_t)q * 16 + e] = KC ? id(a, 16 * c + e) : id(16 * c + e, a);
                filled[(size_t)q]++;
            }
    for (int q = 0; q < chunks; ++q)
        if (filled[(size_t)q] != 1) fail("dma8 chunk filled times", q, filled[(size_t)q], ROWS, KC);
    for (int ks = 0; ks < BK / kstep; ++ks)
        for (int rb = 0; rb < ROWS; rb += 32) {
            int got[64][32];
            if (KC) {
                const int kch = kstep / 16;
                for (int lane = 0; lane < 64; ++lane) {
                    const int r = rb + lane % 32;
                    const uint32_t off =
                        (uint32_t)(r * (BK / 16) + (((lane / 32) * fc) ^ swz_kc(r))) * 16u;
                    for (int c = 0; c < fc; ++c) {
                        const uint32_t a = off ^ (uint32_t)(ks * kch * 16) ^ (uint32_t)(16 * c);
                        for (int e = 0; e < 16; ++e) got[lane][16 * c + e] = lds[a + e];
                    }
                }
            } else {
                for (int c = 0; c < fc; ++c)
                    for (int h = 0; h < 2; ++h) {
                        int in[64][8];
                        int off[64];
                        for (int L = 0; L < 64; ++L) {
                            off[L] = tr8_read_offset(L, fc, ks, kstep, c, h, rb, ROWS);
                            if (off[L] % 8 || off[L] < 0 || off[L] + 8 > bytes)
                                fail("tr8 offset", off[L], L, ks, h);
                            for (int e = 0; e < 8; ++e) in[L][e] = lds[(size_t)off[L] + e];
                        }
                        for (int half = 0; half < 2; ++half) {
                            int used[64] = {0};
                            for (int L = 32 * half; L < 32 * half + 32; ++L)
                                for (int d = 0; d < 2; ++d) used[(off[L] / 4 + d) % 64]++;
                            for (int b = 0; b < 64; ++b)
                                if (used[b] != 1) fail("tr8 bank use", b, used[b], ks, rb);
                        }
                        // the instruction's exchange: lane j element f <- lane
                        // 16*(j/16) + 2f + (j%16)/8, byte j%8
                        for (int j = 0; j < 64; ++j)
                            for (int f = 0; f < 8; ++f)
                                got[j][16 * c + 8 * h + f] =
                                    in[16 * (j / 16) + 2 * f + (j % 16) / 8][j % 8];
                    }
            }
            for (int lane = 0; lane < 64; ++lane)
                for (int c = 0; c < fc; ++c)
                    for (int e = 0; e < 16; ++e) {
                        const int r = rb + lane % 32;
                        const int k = ks * kstep + 16 * fc * (lane / 32) + 16 * c + e;
                        ++g_checked;
                        if (got[lane][16 * c + e] != id(r, k)) fail("fragment8 value", lane, e, r, k);
                    }
        }
}

// The DMA kernels' global side: every lane's 16-byte load of every DMA
// instruction, tile, K slice and K-tile, composed as DmaOperand does
// (init + issue, the clamped form when clampk), must lie inside the
// operand's 16-byte range and hold one of its elements, and an in-range
// chunk must be the one its LDS slot expects.
static void check_dma_global(int ROWS, int BK, int ES, int MF, bool KC, int nwaves, int R, int K,
                             int64_t ld, int kps, bool clampk) {
    const int bytes = ROWS * BK * ES, ni = bytes / 1024 / nwaves, epc = 16 / ES;
    const int ch = BK * ES / 16, chr = ROWS * ES / 16;
    const int64_t range = KC ? operand_range(R, K, ld, ES) : operand_range(K, R, ld, ES);
    const int splits = (K + kps - 1) / kps;
    for (int r0 = 0; r0 < R; r0 += ROWS)
        for (int z = 0; z < splits; ++z) {
            const int kbeg = z * kps, kend = K < kbeg + kps ? K : kbeg + kps;
            for (int k0 = kbeg; k0 < kend; k0 += BK)
                for (int q = 0; q < nwaves * ni * 64; ++q) {
                    int a, c;
                    int64_t off;
                    int row, k;  // the element the chunk starts with, unclamped
                    if (KC) {
                        dma_kc_source(q, ch, a, c);
                        const int64_t voff = kc_chunk_offset(r0 + a, clampk ? 0 : epc * c, R, 1, ld,
                                                             ES, false);
                        off = clampk ? voff + kc_k_offset(k0 + epc * c, kend, ES) : voff + (int64_t)k0 * ES;
                        row = r0 + a;
                        k = k0 + epc * c;
                    } else {
                        if (ES == 2) dma_rc_source(q, chr, MF, a, c); else dma_rc8_source(q, chr, a, c);
                        const int r = r0 + epc * c;
                        const int64_t voff = ES == 2 ? rc_chunk_offset(r, clampk ? 0 : a, R, 1, ld, false)
                                                     : rc8_chunk_offset(r, clampk ? 0 : a, R, 1, ld, false);
                        off = clampk ? voff + (int64_t)imin(k0 + a, kend - 1) * ld * ES
                                     : voff + (int64_t)k0 * ld * ES;
                        row = r;
                        k = k0 + a;
                    }
                    ++g_checked;
                    if (off < 0 || off % 16 != 0 || off + 16 > range)
                        fail("dma load out of range", off, range, row, k);
                    const int64_t line = off / (ld * ES), first = (off % (ld * ES)) / ES;
                    if (line >= (KC ? R : K) || first >= (KC ? K : R))
                        fail("dma chunk holds no element", off, line, first, ES);
                    if (row < R && k < kend) {
                        const int64_t want = KC ? ((int64_t)row * ld + k) * ES : ((int64_t)k * ld + row) * ES;
                        if (off != want) fail("dma wrong chunk", off, want, row, k);
                    }
                }
        }
}

// raster_tile must hit every tile of the grid exactly once.
static void check_raster(int tiles_m, int tiles_n, int group_m, int xcds, int skew) {
    const int T = tiles_m * tiles_n;
    std::vector<int> hits((size_t)T, 0);
    for (int w = 0; w < T; ++w) {
        int tm = -1, tn = -1;
        libgemm::raster_tile(w, tiles_m, tiles_n, group_m, xcds, skew, tm, tn);
        ++g_checked;
        if (tm < 0 || tm >= tiles_m || tn < 0 || tn >= tiles_n) {
            fail("raster tile out of the grid", w, tm, tn, group_m);
            continue;
        }
        ++hits[(size_t)tm * tiles_n + tn];
    }
    for (int i = 0; i < T; ++i)
        if (hits[(size_t)i] != 1) fail("raster tile not hit once", i, hits[(size_t)i], tiles_m, tiles_n);
}

int main() {
    // (R, K, ld) problem sides: the HGEMM workload (A 3999 x 4104 lda 4104, B
    // row-major 4104 x 4001 ldb 4008), ragged small shapes, K below one tile,
    // and a split-K skinny side
    struct Side { int R, K; int64_t ld; int kps; };
    const Side kc_sides[] = {{3999, 4104, 4104, 4160}, {4001, 4104, 4112, 4160}, {37, 77, 80, 128},
                             {13, 1100, 1104, 1152}, {65, 9, 16, 64}, {300, 129, 136, 192},
                             {16, 16384, 16384, 2048}, {16, 1000, 1008, 256}};
    // tiles (ROWS, BK, THREADS) of the table's entries, 16-bit then 8-bit
    const int tiles16[][3] = {{256, 64, 512}, {256, 64, 256}, {128, 64, 256}, {64, 64, 256},
                              {16, 128, 256}, {128, 128, 256}};
    const int tiles8[][3] = {{256, 128, 512}, {256, 128, 256}, {128, 128, 256}, {64, 128, 256},
                             {16, 256, 256}, {128, 256, 256}};
    for (const Side &s : kc_sides) {
        for (const auto &t : tiles16) {
            const int kps = ((s.kps + t[1] - 1) / t[1]) * t[1];
            check_kc(t[0], t[1], t[2], 2, s.R, s.K, s.ld, kps);
            check_rc(t[0], t[1], t[2], s.R, s.K, (s.R + 7) / 8 * 8 + 8, kps);
        }
        for (const auto &t : tiles8) {
            const int kps = ((s.kps + t[1] - 1) / t[1]) * t[1];
            check_kc(t[0], t[1], t[2], 1, s.R, s.K, (s.ld + 15) / 16 * 16, kps);
            check_rc8(t[0], t[1], t[2], s.R, s.K, (s.R + 15) / 16 * 16, kps);
            check_rc8(t[0], t[1], t[2], s.R, s.K, (s.R + 15) / 16 * 16 + 16, kps);
        }
    }
    // R-contiguous B of the HGEMM workload exactly: 4001 columns, ldb 4008
    check_rc(256, 64, 512, 4001, 4104, 4008, 4160);
    check_rc(256, 64, 256, 4001, 4104, 4008, 4160);
    // the DMA kernels' tiles: 256 rows, BK 64, 4 or 8 waves, both MFMA
    // shapes, both storage orders
    for (int nw : {4, 8})
        for (int mf : {32, 16})
            for (bool kc : {true, false}) check_dma_tile(256, 64, mf, kc, nw);
    for (int nw : {4, 8}) check_dma_tile(256, 64, 16, true, nw, true);
    // the 16x16 lane-group order: a permutation, groups g and g + 2 (which
    // read the same rows) at chunks of opposite parity
    {
        int seen = 0;
        for (int g = 0; g < 4; ++g) {
            seen |= 1 << kc_group16(g);
            ++g_checked;
            if (g < 2 && ((kc_group16(g) ^ kc_group16(g + 2)) & 1) != 1) fail("kc_group16 parity", g, 0, 0, 0);
        }
        if (seen != 15) fail("kc_group16 permutation", seen, 0, 0, 0);
    }
    // the DMA loads' global offsets over the problem sides above (16-byte
    // lines as the DMA entries require), 16-bit and 8-bit, both orders, the
    // plain and the clamped form
    for (const Side &s : kc_sides)
        for (int es : {2, 1})
            for (bool kc : {true, false}) {
                const int bk = 128 / es;
                const int kps = ((s.kps + bk - 1) / bk) * bk;
                const bool ragged = (s.K % bk) != 0 || (kps % bk) != 0;
                const int inner = kc ? s.K : s.R;
                const int64_t ld = ((int64_t)inner * es + 15) / 16 * 16 / es + (kc ? 0 : 16 / es);
                for (int nw : {4, 8})
                    for (bool clampk : {true, false}) {
                        if (!clampk && ragged) continue;  // the kernels clamp whenever K is ragged
                        if (es == 1 && nw == 4) continue;
                        check_dma_global(256, bk, es, 32, kc, nw, s.R, s.K, ld, kps, clampk);
                    }
            }
    // the 8-bit DMA tiles: 256 rows x 128 bytes, eight waves, int8 (one
    // chunk per lane) and fp8 (two), both storage orders
    for (int fc : {1, 2})
        for (bool kc : {true, false}) check_dma_tile8(256, 128, fc, kc, 8);
    // the raster: grids of one tile to several rounds per CU, ragged groups,
    // every group height and XCD count the host uses, with and without skew
    const int grids[][2] = {{1, 1}, {1, 7}, {7, 1}, {16, 16}, {64, 64}, {63, 65}, {5, 33}, {32, 32}, {3, 200}};
    for (const auto &gd : grids)
        for (int gm : {1, 2, 4, 8})
            for (int nx : {1, 2, 8})
                for (int sk : {0, 1}) check_raster(gd[0], gd[1], gm, nx, sk);
    printf("checked %ld chunk reads and raster tiles, %ld failures\n", g_checked, g_fail);
    return g_fail ? 1 : 0;
}
