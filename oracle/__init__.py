"""CPU oracle for D = A x B + C (fp64 accumulation, one rounding to the output dtype).

TEST INFRASTRUCTURE ONLY: the test suite, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` are the only callers.  The GPU library
(``dense_mixed_precision_tiled_amd``) neither imports this package nor links its
C code, and this package imports nothing from it.

The arithmetic lives in ``gemm_oracle.c`` (plain C, built with gcc
``-O2 -ffp-contract=off``); this module only builds it and marshals numpy
arrays through ctypes.  Definitions followed (page title, section):

* element definition, ``C[i,j] = sum_k A[i,k] * B[k,j]``:
  "矩阵乘法优化可视化学习文档" section 1, with the triple loop of section 3;
* ``D = A*B + C``, D in the precision of C:
  "深入CUDA Tensor Core与WMMA…" section 2.2;
* row/col-major addressing with a leading dimension:
  same page sections 3.2 and 4.2;
* in-place ``C = A*B + C`` and saturate-to-finite:
  "CUDA算子优化(5)：WMMA矩阵乘法" section "WMMA API解释" item (5);
* OCP fp8 inputs (E4M3, E5M2; one byte per element) in every float function;
* int8 x int8 -> int32 (``gemm_i8``): the type lists of
  "CUDA算子优化(5)：WMMA矩阵乘法" and "深入CUDA Tensor Core与WMMA…" section 2.3;
* the extended epilogue ``D = act(alpha*(A x B) + beta*C + bias)`` with row- or
  column-major C and D (``gemm_ex``): "矩阵乘法优化可视化学习文档" section 6
  (epilogue fusion) and section 8 (bias/activation at the final store), and the
  accumulator layouts of "CUDA算子优化(5)：WMMA矩阵乘法" section "WMMA API解释"
  items (3) and (4);
* the product form (``gemm_product``, ``gemm_i8_product``) of the same
  definitions for whole outputs of large problems: the operands decoded
  exactly to fp64, their product formed by numpy's fp64 matmul (a library
  step), then the C epilogue, single rounding and satf above.

Every function here is pinned by ``tests/test_oracle_pins.py`` against values
and properties the pages and the mathematics fix (no GPU involved).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "gemm_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

# dtype and layout codes (the same integers the C-ABI library uses; the values
# are part of the call contract, not shared code)
F32, F16, BF16 = 0, 1, 2
ROW_MAJOR, COL_MAJOR = 0, 1
ACT_NONE, ACT_RELU, ACT_GELU = 0, 1, 2
I8, I32 = 3, 4
FP8_E4M3, FP8_E5M2 = 5, 6

_lib = None


def build(force: bool = True) -> str:
    """Compile gemm_oracle.c into liboracle.so with gcc (host only); without
    force, only when the library is missing or older than the source."""
    stale = not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC)
    if force or stale:
        tmp = LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math",
               "-fPIC", "-shared", "-pthread", SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, LIB)
    return LIB


def _load():
    global _lib
    if _lib is None:
        build(force=False)
        lib = ctypes.CDLL(LIB)
        i64, vp, c_int = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int
        lib.oracle_gemm.restype = c_int
        lib.oracle_gemm.argtypes = [i64, i64, i64, vp, i64, c_int, vp, i64, c_int,
                                    vp, i64, vp, i64, c_int, c_int, c_int, c_int, c_int]
        lib.oracle_gemm_sampled.restype = c_int
        lib.oracle_gemm_sampled.argtypes = [i64, i64, i64, vp, i64, c_int, vp, i64, c_int,
                                            vp, i64, i64, vp, vp, vp,
                                            c_int, c_int, c_int, c_int, c_int]
        lib.oracle_element_fp64.restype = ctypes.c_double
        lib.oracle_element_fp64.argtypes = [i64, vp, i64, c_int, vp, i64, c_int, vp, i64,
                                            c_int, c_int, i64, i64]
        dbl, fp = ctypes.c_double, ctypes.c_void_p
        lib.oracle_gemm_ex.restype = c_int
        lib.oracle_gemm_ex.argtypes = [i64, i64, i64, vp, i64, c_int, vp, i64, c_int,
                                       vp, i64, c_int, vp, i64, c_int,
                                       c_int, c_int, c_int, c_int, dbl, dbl, fp, c_int, c_int]
        lib.oracle_gemm_ex_sampled.restype = c_int
        lib.oracle_gemm_ex_sampled.argtypes = [i64, i64, i64, vp, i64, c_int, vp, i64, c_int,
                                               vp, i64, c_int, i64, vp, vp, vp,
                                               c_int, c_int, c_int, c_int, dbl, dbl, fp, c_int,
                                               c_int]
        lib.oracle_element_ex_fp64.restype = dbl
        lib.oracle_element_ex_fp64.argtypes = [i64, vp, i64, c_int, vp, i64, c_int,
                                               vp, i64, c_int, c_int, c_int, dbl, dbl, fp,
                                               c_int, i64, i64]
        lib.oracle_gemm_i8.restype = c_int
        lib.oracle_gemm_i8.argtypes = [i64, i64, i64, vp, i64, c_int, vp, i64, c_int,
                                       vp, i64, c_int, vp, i64, c_int, c_int, c_int]
        lib.oracle_gemm_i8_sampled.restype = c_int
        lib.oracle_gemm_i8_sampled.argtypes = [i64, i64, i64, vp, i64, c_int, vp, i64, c_int,
                                               vp, i64, c_int, i64, vp, vp, vp, c_int, c_int]
        lib.oracle_activation.restype = dbl
        lib.oracle_activation.argtypes = [dbl, c_int]
        lib.oracle_decode_fp8_e4m3.restype = ctypes.c_double
        lib.oracle_decode_fp8_e4m3.argtypes = [ctypes.c_uint8]
        lib.oracle_decode_fp8_e5m2.restype = ctypes.c_double
        lib.oracle_decode_fp8_e5m2.argtypes = [ctypes.c_uint8]
        lib.oracle_decode_f16.restype = ctypes.c_double
        lib.oracle_decode_f16.argtypes = [ctypes.c_uint16]
        lib.oracle_decode_bf16.restype = ctypes.c_double
        lib.oracle_decode_bf16.argtypes = [ctypes.c_uint16]
        lib.oracle_round_f16.restype = ctypes.c_uint16
        lib.oracle_round_f16.argtypes = [ctypes.c_double]
        lib.oracle_round_bf16.restype = ctypes.c_uint16
        lib.oracle_round_bf16.argtypes = [ctypes.c_double]
        lib.oracle_round_f32_bits.restype = ctypes.c_uint32
        lib.oracle_round_f32_bits.argtypes = [ctypes.c_double]
        lib.oracle_decode_array.restype = c_int
        lib.oracle_decode_array.argtypes = [c_int, vp, i64, vp]
        lib.oracle_finish_array.restype = c_int
        lib.oracle_finish_array.argtypes = [i64, i64, vp, vp, i64, c_int, vp, i64, c_int,
                                            c_int, c_int, dbl, dbl, fp, c_int, c_int]
        lib.oracle_finish_i8_array.restype = c_int
        lib.oracle_finish_i8_array.argtypes = [i64, i64, vp, vp, i64, c_int, vp, i64, c_int,
                                               c_int]
        _lib = lib
    return _lib


def default_threads() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return max(1, os.cpu_count() or 1)


def _ptr(a):
    return None if a is None else a.ctypes.data


def _check_in(a):
    if a.dtype not in (np.uint16, np.uint8) or not a.flags.c_contiguous:
        raise TypeError("A/B must be C-contiguous bit patterns (uint16, or uint8 for fp8)")


def _check_out(a, out_dtype):
    want = np.float32 if out_dtype == F32 else np.uint16
    if a.dtype != want or not a.flags.c_contiguous:
        raise TypeError("C/D must be C-contiguous %s" % np.dtype(want).name)


def gemm(M, N, K, A, lda, layoutA, B, ldb, layoutB, C, ldc, D, ldd,
         in_dtype, acc_dtype, out_dtype, satf, nthreads=None):
    """D = A x B + C on flat buffers (numpy), same argument order as gemm_run.

    A and B hold 16-bit patterns (uint16) of ``in_dtype``; C and D hold
    ``out_dtype`` elements (float32, or uint16 patterns).  ``C`` may be None
    (C = 0) or the same array as ``D`` with ``ldc == ldd`` (in place).  Only
    ``D[i*ldd + j]`` with i < M, j < N is written.
    """
    _check_in(A)
    _check_in(B)
    _check_out(D, out_dtype)
    if C is not None:
        _check_out(C, out_dtype)
    nt = default_threads() if nthreads is None else nthreads
    rc = _load().oracle_gemm(M, N, K, _ptr(A), lda, layoutA, _ptr(B), ldb, layoutB,
                             _ptr(C), ldc, _ptr(D), ldd,
                             in_dtype, acc_dtype, out_dtype, int(bool(satf)), nt)
    if rc != 0:
        raise ValueError("oracle_gemm rejected its arguments")
    return D


def gemm_sampled(M, N, K, A, lda, layoutA, B, ldb, layoutB, C, ldc, rows, cols,
                 in_dtype, acc_dtype, out_dtype, satf, nthreads=None):
    """Return D(rows[s], cols[s]) for every s as a dense out_dtype array."""
    _check_in(A)
    _check_in(B)
    if C is not None:
        _check_out(C, out_dtype)
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    cols = np.ascontiguousarray(cols, dtype=np.int64)
    if rows.shape != cols.shape:
        raise ValueError("rows and cols differ in length")
    out = np.empty(rows.shape, dtype=np.float32 if out_dtype == F32 else np.uint16)
    nt = default_threads() if nthreads is None else nthreads
    rc = _load().oracle_gemm_sampled(M, N, K, _ptr(A), lda, layoutA, _ptr(B), ldb, layoutB,
                                     _ptr(C), ldc, rows.size, _ptr(rows), _ptr(cols),
                                     _ptr(out), in_dtype, acc_dtype, out_dtype,
                                     int(bool(satf)), nt)
    if rc != 0:
        raise ValueError("oracle_gemm_sampled rejected its arguments")
    return out


def element_fp64(K, A, lda, layoutA, B, ldb, layoutB, C, ldc, in_dtype, out_dtype, i, j):
    """The fp64 value of sum_k A(i,k)B(k,j) (+ C[i,j]) before the final rounding."""
    return _load().oracle_element_fp64(K, _ptr(A), lda, layoutA, _ptr(B), ldb, layoutB,
                                       _ptr(C), ldc, in_dtype, out_dtype, i, j)


def decode_fp8_e4m3(bits: int) -> float:
    return _load().oracle_decode_fp8_e4m3(bits)


def decode_fp8_e5m2(bits: int) -> float:
    return _load().oracle_decode_fp8_e5m2(bits)


def decode_f16(bits: int) -> float:
    return _load().oracle_decode_f16(bits)


def decode_bf16(bits: int) -> float:
    return _load().oracle_decode_bf16(bits)


def round_f16(x: float) -> int:
    return _load().oracle_round_f16(x)


def round_bf16(x: float) -> int:
    return _load().oracle_round_bf16(x)


def round_f32_bits(x: float) -> int:
    return _load().oracle_round_f32_bits(x)


def _check_bias(bias, N):
    if bias is None:
        return None
    if bias.dtype != np.float32 or not bias.flags.c_contiguous or bias.size < N:
        raise TypeError("bias must be a C-contiguous float32 array of at least N values")
    return bias


def gemm_ex(M, N, K, A, lda, layoutA, B, ldb, layoutB, C, ldc, layoutC, D, ldd, layoutD,
            in_dtype, acc_dtype, out_dtype, satf, alpha=1.0, beta=1.0, bias=None,
            act=ACT_NONE, nthreads=None):
    """D = act(alpha * A x B + beta * C + bias) with row/col-major C and D.

    ``bias`` is None or N float32 values (one per column); ``beta == 0``
    means C is not read.  Only D(i, j) with i < M, j < N is written.
    """
    _check_in(A)
    _check_in(B)
    _check_out(D, out_dtype)
    if C is not None:
        _check_out(C, out_dtype)
    bias = _check_bias(bias, N)
    nt = default_threads() if nthreads is None else nthreads
    rc = _load().oracle_gemm_ex(M, N, K, _ptr(A), lda, layoutA, _ptr(B), ldb, layoutB,
                                _ptr(C), ldc, layoutC, _ptr(D), ldd, layoutD,
                                in_dtype, acc_dtype, out_dtype, int(bool(satf)),
                                float(alpha), float(beta), _ptr(bias), int(act), nt)
    if rc != 0:
        raise ValueError("oracle_gemm_ex rejected its arguments")
    return D


def gemm_ex_sampled(M, N, K, A, lda, layoutA, B, ldb, layoutB, C, ldc, layoutC, rows, cols,
                    in_dtype, acc_dtype, out_dtype, satf, alpha=1.0, beta=1.0, bias=None,
                    act=ACT_NONE, nthreads=None):
    """D(rows[s], cols[s]) of gemm_ex for every s, as a dense out_dtype array."""
    _check_in(A)
    _check_in(B)
    if C is not None:
        _check_out(C, out_dtype)
    bias = _check_bias(bias, N)
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    cols = np.ascontiguousarray(cols, dtype=np.int64)
    if rows.shape != cols.shape:
        raise ValueError("rows and cols differ in length")
    out = np.empty(rows.shape, dtype=np.float32 if out_dtype == F32 else np.uint16)
    nt = default_threads() if nthreads is None else nthreads
    rc = _load().oracle_gemm_ex_sampled(M, N, K, _ptr(A), lda, layoutA, _ptr(B), ldb, layoutB,
                                        _ptr(C), ldc, layoutC, rows.size, _ptr(rows),
                                        _ptr(cols), _ptr(out), in_dtype, acc_dtype, out_dtype,
                                        int(bool(satf)), float(alpha), float(beta), _ptr(bias),
                                        int(act), nt)
    if rc != 0:
        raise ValueError("oracle_gemm_ex_sampled rejected its arguments")
    return out


def element_ex_fp64(K, A, lda, layoutA, B, ldb, layoutB, C, ldc, layoutC, in_dtype, out_dtype,
                    alpha, beta, bias, act, i, j):
    """fp64 value of one gemm_ex element after the activation, before rounding."""
    return _load().oracle_element_ex_fp64(K, _ptr(A), lda, layoutA, _ptr(B), ldb, layoutB,
                                          _ptr(C), ldc, layoutC, in_dtype, out_dtype,
                                          float(alpha), float(beta), _ptr(bias), int(act), i, j)


def activation(x: float, act: int) -> float:
    """The oracle's activation function alone (fp64)."""
    return _load().oracle_activation(x, act)


def _check_i8(a):
    if a.dtype != np.int8 or not a.flags.c_contiguous:
        raise TypeError("A/B must be C-contiguous int8 arrays")


def _check_i32(a):
    if a.dtype != np.int32 or not a.flags.c_contiguous:
        raise TypeError("C/D must be C-contiguous int32 arrays")


def gemm_i8(M, N, K, A, lda, layoutA, B, ldb, layoutB, C, ldc, layoutC, D, ldd, layoutD,
            satf, nthreads=None):
    """D = to_int32(A x B + C) for int8 A, B and int32 C, D: the exact sum,
    wrapped modulo 2^32, or clamped to the int32 range with satf."""
    _check_i8(A)
    _check_i8(B)
    _check_i32(D)
    if C is not None:
        _check_i32(C)
    nt = default_threads() if nthreads is None else nthreads
    rc = _load().oracle_gemm_i8(M, N, K, _ptr(A), lda, layoutA, _ptr(B), ldb, layoutB,
                                _ptr(C), ldc, layoutC, _ptr(D), ldd, layoutD,
                                int(bool(satf)), nt)
    if rc != 0:
        raise ValueError("oracle_gemm_i8 rejected its arguments")
    return D


def gemm_i8_sampled(M, N, K, A, lda, layoutA, B, ldb, layoutB, C, ldc, layoutC, rows, cols,
                    satf, nthreads=None):
    """D(rows[s], cols[s]) of gemm_i8 for every s (int32)."""
    _check_i8(A)
    _check_i8(B)
    if C is not None:
        _check_i32(C)
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    cols = np.ascontiguousarray(cols, dtype=np.int64)
    out = np.empty(rows.shape, dtype=np.int32)
    nt = default_threads() if nthreads is None else nthreads
    rc = _load().oracle_gemm_i8_sampled(M, N, K, _ptr(A), lda, layoutA, _ptr(B), ldb, layoutB,
                                        _ptr(C), ldc, layoutC, rows.size, _ptr(rows),
                                        _ptr(cols), _ptr(out), int(bool(satf)), nt)
    if rc != 0:
        raise ValueError("oracle_gemm_i8_sampled rejected its arguments")
    return out


# ------------------------------------------------------------- product form

def decode_array(X, dtype: int) -> np.ndarray:
    """All elements of the flat array X (16-bit patterns, int8, fp8 bytes,
    float32 or int32) decoded exactly to float64 by the C decoders."""
    X = np.ascontiguousarray(X)
    out = np.empty(X.size, dtype=np.float64)
    if _load().oracle_decode_array(int(dtype), X.ctypes.data, X.size, out.ctypes.data) != 0:
        raise ValueError("oracle_decode_array: unknown dtype %r" % dtype)
    return out


def _matrix(X, dtype, rows, cols, ld, layout) -> np.ndarray:
    """The rows x cols matrix X(r, c) held in flat X (row-major: X[r*ld + c],
    column-major: X[c*ld + r]), decoded to float64."""
    outer, inner = (rows, cols) if layout == ROW_MAJOR else (cols, rows)
    if rows == 0 or cols == 0:
        return np.zeros((rows, cols))
    flat = np.ascontiguousarray(X).ravel()
    need = (outer - 1) * ld + inner
    if flat.size < need or ld < inner:
        raise ValueError("operand buffer too small for its shape and leading dimension")
    v = decode_array(flat[:need], dtype)
    v = np.concatenate([v, np.zeros(outer * ld - need)]).reshape(outer, ld)[:, :inner]
    return v if layout == ROW_MAJOR else v.T


def product_sums(M, N, K, A, lda, layoutA, B, ldb, layoutB, in_dtype) -> np.ndarray:
    """S(i, j) = sum_k A(i, k) * B(k, j) in fp64 as an M x N dense array: the
    exactly decoded operands multiplied by numpy's fp64 matmul.  Exact where
    every partial sum is (integer-valued inputs); otherwise within fp64
    rounding, about K * 2^-53 * sum_k |A(i,k) * B(k,j)|."""
    if K == 0 or M == 0 or N == 0:
        return np.zeros((M, N))
    a = _matrix(A, in_dtype, M, K, lda, layoutA)
    b = _matrix(B, in_dtype, K, N, ldb, layoutB)
    return np.ascontiguousarray(a @ b)


def gemm_product(M, N, K, A, lda, layoutA, B, ldb, layoutB, C, ldc, D, ldd,
                 in_dtype, acc_dtype, out_dtype, satf, layoutC=ROW_MAJOR, layoutD=ROW_MAJOR,
                 alpha=1.0, beta=1.0, bias=None, act=ACT_NONE, nthreads=None, sums=None):
    """gemm / gemm_ex for whole outputs of large problems: the sums from
    ``product_sums`` (or the given ``sums``), then the epilogue, one rounding
    and satf of the C oracle.  Same arguments and results as ``gemm_ex``
    (C == D in place; only D(i, j) with i < M, j < N written), up to the fp64
    summation order (see product_sums); ``acc_dtype`` only names the call."""
    del acc_dtype
    _check_in(A)
    _check_in(B)
    _check_out(D, out_dtype)
    if C is not None:
        _check_out(C, out_dtype)
    bias = _check_bias(bias, N)
    S = product_sums(M, N, K, A, lda, layoutA, B, ldb, layoutB, in_dtype) if sums is None \
        else np.ascontiguousarray(sums, dtype=np.float64)
    nt = default_threads() if nthreads is None else nthreads
    rc = _load().oracle_finish_array(M, N, _ptr(S), _ptr(C), ldc, layoutC, _ptr(D), ldd,
                                     layoutD, out_dtype, int(bool(satf)), float(alpha),
                                     float(beta), _ptr(bias), int(act), nt)
    if rc != 0:
        raise ValueError("oracle_finish_array rejected its arguments")
    return D


def gemm_i8_product(M, N, K, A, lda, layoutA, B, ldb, layoutB, C, ldc, layoutC, D, ldd,
                    layoutD, satf):
    """gemm_i8 for whole outputs of large problems: the int8 operands as exact
    fp64 values, their fp64 matmul (exact while K < 2^39, every partial sum
    below 2^53), then + C and the wrap or clamp to int32 of the C oracle."""
    _check_i8(A)
    _check_i8(B)
    _check_i32(D)
    if C is not None:
        _check_i32(C)
    if K >= 2 ** 39:
        raise ValueError("gemm_i8_product: fp64 sums are exact only for K < 2^39")
    S = product_sums(M, N, K, A, lda, layoutA, B, ldb, layoutB, I8)
    rc = _load().oracle_finish_i8_array(M, N, _ptr(S), _ptr(C), ldc, layoutC, _ptr(D), ldd,
                                        layoutD, int(bool(satf)))
    if rc != 0:
        raise ValueError("oracle_finish_i8_array rejected its arguments")
    return D
