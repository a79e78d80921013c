"""Pins of the oracle's int8 x int8 -> int32 GEMM against Python integers.

No GPU.  Python's unbounded ints give the exact sum; wrapping modulo 2^32 and
clamping to the int32 range are written out here independently of the C code.
"""
import itertools

import numpy as np
import pytest

import oracle

ROW, COL = oracle.ROW_MAJOR, oracle.COL_MAJOR
I32_MIN, I32_MAX = -2 ** 31, 2 ** 31 - 1


@pytest.fixture(scope="module", autouse=True)
def _built():
    oracle.build(force=False)


def wrap32(v: int) -> int:
    return ((v + 2 ** 31) % 2 ** 32) - 2 ** 31


def clamp32(v: int) -> int:
    return min(max(v, I32_MIN), I32_MAX)


def _at(layout, ld, r, c):
    return r * ld + c if layout == ROW else c * ld + r


CASES = list(itertools.product([(1, 1, 1), (2, 3, 4), (3, 2, 6), (4, 5, 0)],
                               [ROW, COL], [ROW, COL], [ROW, COL], [ROW, COL], [0, 1],
                               ["none", "sep", "big"]))


@pytest.mark.parametrize("shape,la,lb,lc,ld,satf,cmode",
                         [c for n, c in enumerate(CASES) if n % 3 == 0])
def test_bruteforce_vs_python_integers(shape, la, lb, lc, ld, satf, cmode):
    M, N, K = shape
    rng = np.random.default_rng(hash((shape, la, lb, lc, ld, satf, cmode)) % 2 ** 32)
    lda = (K if la == ROW else M) + 1
    ldb = (N if lb == ROW else K) + 2
    A = rng.integers(-128, 128, size=(M if la == ROW else K) * lda, dtype=np.int64).astype(np.int8)
    B = rng.integers(-128, 128, size=(K if lb == ROW else N) * ldb, dtype=np.int64).astype(np.int8)
    ldc = (N if lc == ROW else M) + 1
    C = None
    if cmode != "none":
        lo, hi = ((I32_MIN, I32_MAX) if cmode == "big" else (-1000, 1000))
        C = rng.integers(lo, hi, size=(M if lc == ROW else N) * ldc, dtype=np.int64,
                         endpoint=True).astype(np.int32)
    ldd = (N if ld == ROW else M) + 3
    D = np.full((M if ld == ROW else N) * ldd + 5, 0x5A5A5A5A, dtype=np.int32)
    oracle.gemm_i8(M, N, K, A, lda, la, B, ldb, lb, C, ldc, lc, D, ldd, ld, satf)
    written = set()
    for i in range(M):
        for j in range(N):
            s = sum(int(A[_at(la, lda, i, k)]) * int(B[_at(lb, ldb, k, j)]) for k in range(K))
            if C is not None:
                s += int(C[_at(lc, ldc, i, j)])
            want = clamp32(s) if satf else wrap32(s)
            off = _at(ld, ldd, i, j)
            written.add(off)
            assert int(D[off]) == want, (i, j, s, int(D[off]), want)
    assert all(int(D[o]) == 0x5A5A5A5A for o in range(D.size) if o not in written)


def test_every_byte_pattern_decodes_as_twos_complement():
    A = np.arange(256, dtype=np.uint8).view(np.int8).copy()   # column vector, 256 x 1
    B = np.ones(1, dtype=np.int8)
    D = np.zeros(256, dtype=np.int32)
    oracle.gemm_i8(256, 1, 1, A, 1, ROW, B, 1, ROW, None, 1, ROW, D, 1, ROW, 0)
    assert [int(x) for x in D] == [b - 256 if b >= 128 else b for b in range(256)]


@pytest.mark.parametrize("satf", [0, 1])
def test_overflow_through_a_long_sum(satf):
    """K = 140000 products of 127*127 (and of -128*127) leave the int32 range:
    the wrapped and the clamped results differ from the exact sum."""
    K = 140000
    for a, b in ((127, 127), (-128, 127)):
        A = np.full(K, a, dtype=np.int8)
        B = np.full(K, b, dtype=np.int8)
        D = np.zeros(1, dtype=np.int32)
        oracle.gemm_i8(1, 1, K, A, K, ROW, B, 1, ROW, None, 1, ROW, D, 1, ROW, satf)
        exact = K * a * b
        assert abs(exact) > 2 ** 31
        assert int(D[0]) == (clamp32(exact) if satf else wrap32(exact))


def test_in_place_and_sampled():
    rng = np.random.default_rng(4)
    M, N, K = 7, 5, 33
    A = rng.integers(-128, 128, size=M * K).astype(np.int8)
    B = rng.integers(-128, 128, size=K * N).astype(np.int8)
    C = rng.integers(-10 ** 6, 10 ** 6, size=N * M).astype(np.int32)
    ref = np.zeros(N * M, dtype=np.int32)
    oracle.gemm_i8(M, N, K, A, K, ROW, B, N, ROW, C, M, COL, ref, M, COL, 0)
    D = C.copy()
    oracle.gemm_i8(M, N, K, A, K, ROW, B, N, ROW, D, M, COL, D, M, COL, 0)
    assert np.array_equal(D, ref)
    rows, cols = rng.integers(0, M, 20), rng.integers(0, N, 20)
    got = oracle.gemm_i8_sampled(M, N, K, A, K, ROW, B, N, ROW, C, M, COL, rows, cols, 0)
    assert np.array_equal(got, ref.reshape(N, M)[cols, rows])


def test_matches_numpy_int64_matmul():
    rng = np.random.default_rng(5)
    M, N, K = 33, 47, 129
    A = rng.integers(-128, 128, size=(M, K)).astype(np.int8)
    B = rng.integers(-128, 128, size=(N, K)).astype(np.int8)   # column-major K x N
    D = np.zeros(M * N, dtype=np.int32)
    oracle.gemm_i8(M, N, K, A.ravel(), K, ROW, B.ravel(), K, COL, None, N, ROW, D, N, ROW, 0)
    assert np.array_equal(D.reshape(M, N), A.astype(np.int64) @ B.astype(np.int64).T)
