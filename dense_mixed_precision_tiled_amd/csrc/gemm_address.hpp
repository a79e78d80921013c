// Address arithmetic of the 16-byte operand loads, shared by the kernels and
// a host-side check (this header needs no HIP; compiled by a plain C++
// compiler it gives the host functions the CPU test enumerates).
//
// Every vector load reads one 16-byte chunk.  The functions below clamp the
// row and the k position so that each chunk read contains at least one
// element of the operand's matrix: rows past the matrix's last row read the
// last row, and k positions past the last valid k read the chunk that holds
// the last valid k.  Such chunks feed only outputs that are never stored
// (rows) or are masked to zero before use (k), so the clamps change no
// result; they keep every read inside the 16-byte-aligned chunks the matrix
// occupies, independent of the hardware's buffer range check.
#pragma once

#include <stdint.h>

#if defined(__HIPCC__) || defined(__HIP__)
#define LIBGEMM_HD __host__ __device__
#else
#define LIBGEMM_HD
#endif

namespace libgemm {

LIBGEMM_HD inline int imin(int a, int b) { return a < b ? a : b; }
LIBGEMM_HD inline int imax(int a, int b) { return a > b ? a : b; }

// K-contiguous storage, X(r, k) = X[r*ld + k], elements of es bytes, 16/es
// elements per chunk (chunks start at k multiples of 16/es).
//   kc_row_offset: byte offset of row r, clamped to [0, R-1];
//   kc_k_offset:   byte offset of position k inside a row, clamped to the
//                  chunk holding kend-1;
//   kc_chunk_offset: the chunk holding X(r, k..), k clamped when clampk.
LIBGEMM_HD inline int64_t kc_row_offset(int r, int R, int64_t ld, int es) {
    return (int64_t)imin(r, R - 1) * ld * es;
}
LIBGEMM_HD inline int64_t kc_k_offset(int k, int kend, int es) {
    const int epc = 16 / es;
    return (int64_t)imin(k, ((kend - 1) / epc) * epc) * es;
}
LIBGEMM_HD inline int64_t kc_chunk_offset(int r, int k, int R, int kend, int64_t ld, int es,
                                          bool clampk) {
    return kc_row_offset(r, R, ld, es) + (clampk ? kc_k_offset(k, kend, es) : (int64_t)k * es);
}

// R-contiguous storage, X(r, k) = X[k*ld + r] (16-bit elements): byte offset
// of the chunk holding X(r..r+7, k), with the 8-aligned column r clamped to
// the chunk holding column R-1 and, when clampk, k clamped to kend-1.
LIBGEMM_HD inline int64_t rc_chunk_offset(int r, int k, int R, int kend, int64_t ld,
                                          bool clampk) {
    const int rr = imin(r, (R - 1) & ~7);
    const int kk = clampk ? imin(k, kend - 1) : k;
    return ((int64_t)kk * ld + rr) * 2;
}

// R-contiguous storage of 8-bit elements: byte offset of the dword holding
// X(r..r+3, k), with the 4-aligned column r clamped to the dword holding
// column R-1 and, when clampk, k clamped to kend-1.
LIBGEMM_HD inline int64_t rc8_dword_offset(int r, int k, int R, int kend, int64_t ld,
                                           bool clampk) {
    const int rr = imin(r, (R - 1) & ~3);
    const int kk = clampk ? imin(k, kend - 1) : k;
    return (int64_t)kk * ld + rr;
}

// R-contiguous storage of 8-bit elements: byte offset of the 16-byte chunk
// holding X(r..r+15, k), with the 16-aligned column r clamped to the chunk
// holding column R-1 and, when clampk, k clamped to kend-1 (the LDS-DMA
// loads; ld is a multiple of 16 there).
LIBGEMM_HD inline int64_t rc8_chunk_offset(int r, int k, int R, int kend, int64_t ld,
                                           bool clampk) {
    const int rr = imin(r, (R - 1) & ~15);
    const int kk = clampk ? imin(k, kend - 1) : k;
    return (int64_t)kk * ld + rr;
}

// The in-register transpose of an R-contiguous 8-bit block (4 rows x 16
// k-rows, one dword per k-row): dword d of row e's K-contiguous chunk holds
// byte e of the k-rows 4d..4d+3 (a..d), k-row 4d in byte 0.
LIBGEMM_HD inline uint32_t rc8_gather(uint32_t a, uint32_t b, uint32_t c, uint32_t d, int e) {
    const int s = 8 * e;
    return ((a >> s) & 0xffu) | (((b >> s) & 0xffu) << 8) | (((c >> s) & 0xffu) << 16) |
           (((d >> s) & 0xffu) << 24);
}

// The byte extent the vector path allows: the operand's last element, rounded
// up to 16 bytes (outer lines of inner elements at stride ld).
LIBGEMM_HD inline int64_t operand_range(int64_t outer, int64_t inner, int64_t ld, int es) {
    return (((outer - 1) * ld + inner) * es + 15) & ~(int64_t)15;
}

// ------------------------------------------------------ LDS tile layouts
// K-contiguous tile: row r holds the operand's k values of one row (M for
// A, N for B) as 16-byte chunks; chunk c of row r sits at slot c ^ swz_kc(r).
// Eight consecutive rows read at one chunk (the MFMA operand reads), and
// eight rows 8 apart, land in eight different 16-byte bank groups.
LIBGEMM_HD inline int swz_kc(int r) { return (r ^ (r >> 3)) & 7; }

// K-contiguous fragment reads with the 16x16 MFMAs of one chunk per lane
// and step: lane group g = lane / 16 reads chunk kc_group16(g) of the step
// (0, 2, 1, 3) instead of chunk g.  A and B take the same order, so each
// lane still pairs A's and B's values of the same k.  In the natural order
// these reads measured two-way bank conflicts (the conflict counter at half
// the LDS-active cycles) while the 32x32 reads measured none; the
// permutation gives lane groups g and g + 2, which read the same rows, chunks
// of opposite parity, so those rows' reads fall in different halves of the
// banks.
LIBGEMM_HD inline int kc_group16(int g) { return ((g & 1) << 1) | (g >> 1); }

// R-contiguous tile (row-major B or column-major A kept as stored): k-row k
// holds R values as R/8 chunks; chunk c of k-row k sits at slot
// c ^ swz_rc(k, mf).  The transposed operand reads (ds_read_b64_tr_b16) of
// one half-wave then touch distinct banks: with the 32x32 MFMA a half-wave
// reads 4 k-rows x 64 bytes (the XOR moves whole 64-byte groups by k % 4),
// with the 16x16 MFMA 8 k-rows x 32 bytes (32-byte groups by k % 4 and bit 3
// of k).  Needs R >= 128 (16 chunks).
LIBGEMM_HD inline int swz_rc(int k, int mf) {
    return mf == 32 ? (k & 3) << 2 : ((k & 3) | ((k >> 1) & 4)) << 1;
}

// R-contiguous 8-bit tile: k-row k holds R bytes as R/16 chunks; chunk c of
// k-row k sits at slot c ^ swz_rc8(k).  A 16-lane group of the transposed
// reads (ds_read_b64_tr_b8) touches 8 consecutive k-rows at one chunk, and a
// half-wave two adjacent chunks (an even and an odd one); the XOR moves
// whole 32-byte pairs by k % 8, so the half-wave's 16 chunks, 64 banks, are
// distinct.  Needs R >= 256 (16 chunks).
LIBGEMM_HD inline int swz_rc8(int k) { return (k & 7) << 1; }

// Direct global -> LDS loads write 16 bytes per lane to consecutive LDS
// chunks (lane l of an instruction to chunk q0 + l).  The source a lane
// reads is therefore the chunk that belongs at that slot:
//   K-contiguous tile with ch chunks per row: LDS chunk q holds row
//   q / ch, chunk (q % ch) ^ swz_kc(row), i.e. k = that chunk * (16 / es);
//   R-contiguous tile with chr chunks per k-row: LDS chunk q holds k-row
//   q / chr, rows 8 * ((q % chr) ^ swz_rc(k-row)) .. + 7.
LIBGEMM_HD inline void dma_kc_source(int q, int ch, int &row, int &chunk) {
    row = q / ch;
    chunk = (q % ch) ^ swz_kc(row);
}
LIBGEMM_HD inline void dma_rc_source(int q, int chr, int mf, int &krow, int &chunk) {
    krow = q / chr;
    chunk = (q % chr) ^ swz_rc(krow, mf);
}
// (8-bit R-contiguous tile: rows 16 * ((q % chr) ^ swz_rc8(k-row)) .. + 15)
LIBGEMM_HD inline void dma_rc8_source(int q, int chr, int &krow, int &chunk) {
    krow = q / chr;
    chunk = (q % chr) ^ swz_rc8(krow);
}

// Transposed operand read (ds_read_b64_tr_b16) from an R-contiguous tile with
// rowbytes bytes per k-row: in each group of 16 lanes, lane L supplies the
// address of 4 consecutive 16-bit values and lane j of the group receives
// element j % 4 of lane 4f + (j % 16) / 4 as its element f (f = 0..3).  For
// the MFMA operand of rows rb.. (32 or 16 of them, mf) at k step ks (16 or
// 32 k values) and half h (k offset 0 or 4 inside the lane's 8), lane L
// addresses k-row ks*kstep + kgrp + 4h + (L % 16) / 4 at row
// rb + rsub + 4 * (L % 4), where for mf = 32 kgrp = 8 * (L / 32) and
// rsub = 16 * ((L / 16) % 2), for mf = 16 kgrp = 8 * (L / 16) and rsub = 0.
// Then lane j holds the rows' operand values X(rb + j % mf, k) for the 4
// k-values k = ks*kstep + 8 * (j / mf) + 4h + 0..3 the MFMA expects.
LIBGEMM_HD inline int tr_read_offset(int lane, int mf, int ks, int h, int rb, int rowbytes) {
    const int g = lane / 16, f = (lane % 16) / 4, q = lane % 4;
    const int kstep = mf == 32 ? 16 : 32;
    const int kgrp = mf == 32 ? 8 * (g / 2) : 8 * g;
    const int rsub = mf == 32 ? 16 * (g % 2) : 0;
    const int krow = ks * kstep + kgrp + 4 * h + f;
    const int row = rb + rsub + 4 * q;
    return krow * rowbytes + (((row / 8) ^ swz_rc(krow, mf)) * 16) + (row % 8) * 2;
}

// Transposed 8-bit operand read (ds_read_b64_tr_b8) from an R-contiguous
// tile with rowbytes bytes per k-row: in each group of 16 lanes, lane L
// supplies the address of 8 consecutive bytes and lane j of the group
// receives byte j % 8 of lane 2f + (j % 16) / 8 as its element f (f = 0..7;
// probed on the GPU).  For the 32x32 MFMA operand of rows rb..rb+31 (fc
// 16-byte chunks of k per lane, kstep k values per step) at step ks, chunk c
// and half h (k offset 8h inside the chunk), lane L addresses k-row
// ks*kstep + 16*fc*(L / 32) + 16c + 8h + (L % 16) / 2 at row
// rb + 16 * ((L / 16) % 2) + 8 * (L % 2).  Then lane j holds X(rb + j % 32, k)
// for the 8 k-values k = ks*kstep + 16*fc*(j / 32) + 16c + 8h + 0..7, bytes
// 8h..8h+7 of its operand chunk c, as the MFMA expects.
LIBGEMM_HD inline int tr8_read_offset(int lane, int fc, int ks, int kstep, int c, int h, int rb,
                                      int rowbytes) {
    const int krow = ks * kstep + 16 * fc * (lane / 32) + 16 * c + 8 * h + (lane % 16) / 2;
    const int row = rb + 16 * ((lane / 16) % 2) + 8 * (lane % 2);
    return krow * rowbytes + ((row / 16) ^ swz_rc8(krow)) * 16 + row % 16;
}

// Output tile of workgroup w.  The device hands workgroups to its xcds XCDs
// in turn (w % xcds), so the linear tile index t gives each XCD one
// contiguous run of tiles and the XCD's concurrent workgroups run
// neighbouring tiles, which share operand panels in that XCD's L2.  Tiles
// are numbered in raster groups of group_m tile-rows, column by column
// inside a group (row order when group_m is 1).  With skew, group g starts
// at column g * tiles_n / groups and wraps around: groups that run at the
// same time on different XCDs then work on different column bands, so their
// reads of B and their writes of D spread over the memory channels instead
// of all XCDs streaming the same columns.  Every step is a bijection of
// [0, tiles_m * tiles_n), so each tile is computed exactly once.
LIBGEMM_HD inline void raster_tile(int w, int tiles_m, int tiles_n, int group_m, int xcds,
                                   int skew, int &tm, int &tn) {
    const int T = tiles_m * tiles_n;
    const int xcd = w % xcds, local = w / xcds;
    const int per = T / xcds, rem = T % xcds;
    const int t = xcd * per + imin(xcd, rem) + local;
    const int in_group = group_m * tiles_n;
    const int g = t / in_group;
    const int first_m = g * group_m;
    const int gsize = imin(tiles_m - first_m, group_m);
    const int t_in = t - g * in_group;
    tm = first_m + t_in % gsize;
    tn = t_in / gsize;
    if (skew) {
        const int groups = (tiles_m + group_m - 1) / group_m;
        tn += g * tiles_n / groups;  // g * tiles_n <= tiles_m * tiles_n, an int
        if (tn >= tiles_n) tn -= tiles_n;
    }
}

}  // namespace libgemm
