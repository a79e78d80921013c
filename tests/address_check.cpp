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
                            const int rb = b % RCH, kg = b / RCH;
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
        }
    }
    // R-contiguous B of the HGEMM workload exactly: 4001 columns, ldb 4008
    check_rc(256, 64, 512, 4001, 4104, 4008, 4160);
    check_rc(256, 64, 256, 4001, 4104, 4008, 4160);
    printf("checked %ld chunk reads, %ld failures\n", g_checked, g_fail);
    return g_fail ? 1 : 0;
}
