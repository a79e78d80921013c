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

// The byte extent the vector path allows: the operand's last element, rounded
// up to 16 bytes (outer lines of inner elements at stride ld).
LIBGEMM_HD inline int64_t operand_range(int64_t outer, int64_t inner, int64_t ld, int es) {
    return (((outer - 1) * ld + inner) * es + 15) & ~(int64_t)15;
}

}  // namespace libgemm
