"""Pins of the oracle's product form (oracle.gemm_product, gemm_i8_product):
the whole-output oracle of the large workloads.  No GPU.

It forms the fp64 sums with numpy's matmul of the exactly decoded operands
(a library step) and rounds them with the C oracle's epilogue.  Pinned here
against exact rational sums on tiny dyadic inputs (every fp64 partial sum
exact, so the result must be RNE of the exact value), against the
per-element loops of oracle.gemm / gemm_ex / gemm_i8 (bit for bit on inputs
whose sums fp64 holds exactly, within one output ulp elsewhere), and against
the invariants the definitions fix (in place, padding, satf).
"""
import itertools

import numpy as np
import pytest

import oracle
from exact_rne import BF16, F16, F32, rne_bits, satf_bits, value_of_out
from test_oracle_pins import _buffers, _exact_D, _grid_values

ROW, COL = oracle.ROW_MAJOR, oracle.COL_MAJOR
FP8s = (oracle.FP8_E4M3, oracle.FP8_E5M2)


@pytest.fixture(scope="module", autouse=True)
def _built():
    oracle.build(force=False)


def _bits_of(D, out_dt):
    return D.view(np.uint32) if out_dt == F32 else D


CASES = list(itertools.product(
    [(1, 1, 1), (2, 3, 4), (3, 2, 5), (4, 4, 3), (5, 1, 6), (3, 3, 0)],
    [ROW, COL], [ROW, COL], [F16, BF16],
    [(F32, F32), (F32, F16), (F32, BF16), (F16, F16)],
    ["none", "sep", "inplace"], [0, 1]))


@pytest.mark.parametrize("shape,layA,layB,in_dt,accout,cmode,satf",
                         [c for i, c in enumerate(CASES) if i % 6 == 1])
def test_bruteforce_tiny_vs_exact_rational(shape, layA, layB, in_dt, accout, cmode, satf):
    M, N, K = shape
    acc_dt, out_dt = accout
    rng = np.random.default_rng(hash(("product", shape, layA, layB, in_dt, accout, cmode,
                                      satf)) % 2 ** 32)
    A, lda, B, ldb = _buffers(rng, M, N, K, layA, layB, in_dt, int(rng.integers(0, 3)))
    ldd = N + int(rng.integers(0, 3))
    sentinel = np.float32(-777.25) if out_dt == F32 else np.uint16(0x5A5A)
    D = np.full((M + 1) * ldd, sentinel, dtype=np.float32 if out_dt == F32 else np.uint16)
    C, ldc = None, N
    if cmode == "sep":
        ldc = N + 1
        C = np.zeros(M * ldc, dtype=D.dtype)
        C.reshape(M, ldc)[:, :N] = _grid_values(rng, (M, N), out_dt)
    elif cmode == "inplace":
        ldc = ldd
        D.reshape(M + 1, ldd)[:M, :N] = _grid_values(rng, (M, N), out_dt)
        C = D
    exact = _exact_D(M, N, K, A, lda, layA, B, ldb, layB, C, ldc, in_dt, out_dt)
    oracle.gemm_product(M, N, K, A.ravel(), lda, layA, B.ravel(), ldb, layB, C, ldc, D, ldd,
                        in_dt, acc_dt, out_dt, satf)
    Db = _bits_of(D, out_dt).reshape(M + 1, ldd)
    for (i, j), s in exact.items():
        want = rne_bits(s, out_dt)
        if satf:
            want = satf_bits(want, out_dt)
        if s == 0:
            assert value_of_out(D.reshape(M + 1, ldd)[i, j], out_dt) == 0.0
        else:
            assert int(Db[i, j]) == want, (i, j, float(s), hex(int(Db[i, j])), hex(want))
    sbits = int(np.array([sentinel]).view(np.uint32 if out_dt == F32 else np.uint16)[0])
    assert np.all(Db[:M, N:] == sbits) and np.all(Db[M, :] == sbits)


def _operands(rng, M, N, K, layA, layB, in_dt, values, pad=3):
    a_outer, a_inner = (M, K) if layA == ROW else (K, M)
    b_outer, b_inner = (K, N) if layB == ROW else (N, K)
    lda, ldb = a_inner + pad, b_inner + pad

    def make(outer, inner, ld):
        if values == "int":
            v = rng.integers(-2, 3, size=(outer, ld)).astype(np.float32)
        else:
            v = (rng.random((outer, ld)) * 2 - 1).astype(np.float32)
        if in_dt == F16:
            X = v.astype(np.float16).view(np.uint16)
        else:
            X = (v.view(np.uint32) >> 16).astype(np.uint16)
        X[:, inner:] = 0x7E00 if in_dt == F16 else 0x7FC0   # NaN in the padding
        return X

    return make(a_outer, a_inner, lda), lda, make(b_outer, b_inner, ldb), ldb


@pytest.mark.parametrize("layA,layB,in_dt,out_dt,acc_dt,cmode", [
    (ROW, ROW, F16, F32, F32, "none"), (ROW, COL, BF16, F32, F32, "inplace"),
    (COL, ROW, F16, F16, F16, "sep"), (COL, COL, BF16, BF16, F32, "sep"),
    (ROW, ROW, F16, F16, F16, "inplace")])
@pytest.mark.parametrize("values", ["int", "uniform"])
def test_matches_the_per_element_oracle(layA, layB, in_dt, out_dt, acc_dt, cmode, values):
    """Integer-valued inputs: every fp64 partial sum is exact in either order,
    so the product form equals oracle.gemm bit for bit.  Uniform inputs: the
    two fp64 sums differ only by fp64 rounding, so the rounded outputs may
    differ only where the sum lies that close to a rounding boundary of the
    output type -- at most one output ulp, and (at these sizes) essentially
    never."""
    M, N, K = 67, 91, 300
    rng = np.random.default_rng(hash((layA, layB, in_dt, out_dt, cmode, values)) % 2 ** 32)
    A, lda, B, ldb = _operands(rng, M, N, K, layA, layB, in_dt, values)
    odt = np.float32 if out_dt == F32 else np.uint16
    ldd = N + 2
    D0 = np.full(M * ldd, 0x5A5A if out_dt != F32 else -777.25, dtype=odt)
    C, ldc = None, N
    cvals = (rng.standard_normal((M, N)) if values == "uniform"
             else rng.integers(-2, 3, (M, N))).astype(np.float32)
    if out_dt == F16:
        cvals = cvals.astype(np.float16).view(np.uint16)
    elif out_dt == BF16:
        cvals = (cvals.view(np.uint32) >> 16).astype(np.uint16)
    if cmode == "inplace":
        D0.reshape(M, ldd)[:, :N] = cvals
        ldc = ldd
    elif cmode == "sep":
        ldc = N + 1
        C = np.zeros(M * ldc, dtype=odt)
        C.reshape(M, ldc)[:, :N] = cvals
    D1, D2 = D0.copy(), D0.copy()
    oracle.gemm(M, N, K, A.ravel(), lda, layA, B.ravel(), ldb, layB,
                D1 if cmode == "inplace" else C, ldc, D1, ldd, in_dt, acc_dt, out_dt, 0)
    oracle.gemm_product(M, N, K, A.ravel(), lda, layA, B.ravel(), ldb, layB,
                        D2 if cmode == "inplace" else C, ldc, D2, ldd, in_dt, acc_dt, out_dt, 0)
    b1 = _bits_of(D1, out_dt).astype(np.int64)
    b2 = _bits_of(D2, out_dt).astype(np.int64)
    if values == "int":
        assert np.array_equal(b1, b2)
    else:
        diff = np.abs(b1 - b2)          # same sign: bit distance = ulp distance
        assert diff.max() <= 1 and np.count_nonzero(diff) <= 2, np.count_nonzero(diff)
    # padding untouched
    assert np.array_equal(D2.reshape(M, ldd)[:, N:], D0.reshape(M, ldd)[:, N:])


def test_a_transposed_or_short_operand_is_caught():
    """Reading B in the other layout, or dropping the last k, changes the
    product form's result on a non-square case (so the pins above see it)."""
    rng = np.random.default_rng(5)
    M, N, K = 5, 7, 9
    A, lda, B, ldb = _operands(rng, M, N, K, ROW, ROW, F16, "int", pad=0)
    D = np.zeros(M * N, dtype=np.float32)
    ref = oracle.gemm(M, N, K, A.ravel(), lda, ROW, B.ravel(), ldb, ROW, None, N, D.copy(), N,
                      F16, F32, F32, 0)
    good = oracle.gemm_product(M, N, K, A.ravel(), lda, ROW, B.ravel(), ldb, ROW, None, N,
                               D.copy(), N, F16, F32, F32, 0)
    assert np.array_equal(good, ref)
    Bsq = np.ascontiguousarray(np.resize(B, (K, K)))
    swapped = oracle.gemm_product(M, K, K, A.ravel(), lda, ROW, Bsq.ravel(), K, COL, None, K,
                                  np.zeros(M * K, np.float32), K, F16, F32, F32, 0)
    straight = oracle.gemm_product(M, K, K, A.ravel(), lda, ROW, Bsq.ravel(), K, ROW, None, K,
                                   np.zeros(M * K, np.float32), K, F16, F32, F32, 0)
    assert not np.array_equal(swapped, straight)
    short = oracle.gemm_product(M, N, K - 1, A.ravel(), lda, ROW, B.ravel(), ldb, ROW, None, N,
                                D.copy(), N, F16, F32, F32, 0)
    assert not np.array_equal(short, ref)


@pytest.mark.parametrize("act", [oracle.ACT_NONE, oracle.ACT_RELU, oracle.ACT_GELU])
@pytest.mark.parametrize("layC,layD", [(ROW, ROW), (COL, COL), (ROW, COL)])
def test_extended_epilogue_matches_gemm_ex(act, layC, layD):
    """alpha, beta, bias, activation and column-major C/D through the product
    form equal oracle.gemm_ex (integer-valued operands: the sums agree
    exactly, then both run the same epilogue and rounding)."""
    M, N, K = 33, 40, 120
    rng = np.random.default_rng(hash(("ex", act, layC, layD)) % 2 ** 32)
    A, lda, B, ldb = _operands(rng, M, N, K, ROW, COL, F16, "int", pad=1)
    c_outer, c_inner = (M, N) if layC == ROW else (N, M)
    d_outer, d_inner = (M, N) if layD == ROW else (N, M)
    C = rng.standard_normal(c_outer * c_inner).astype(np.float32)
    bias = rng.standard_normal(N).astype(np.float32)
    D0 = np.full(d_outer * (d_inner + 1), -5.5, dtype=np.float32)
    D1, D2 = D0.copy(), D0.copy()
    args = dict(alpha=-0.5, beta=2.0, bias=bias, act=act)
    oracle.gemm_ex(M, N, K, A.ravel(), lda, ROW, B.ravel(), ldb, COL, C, c_inner, layC,
                   D1, d_inner + 1, layD, F16, F32, F32, 0, **args)
    oracle.gemm_product(M, N, K, A.ravel(), lda, ROW, B.ravel(), ldb, COL, C, c_inner, D2,
                        d_inner + 1, F16, F32, F32, 0, layoutC=layC, layoutD=layD, **args)
    assert np.array_equal(D1.view(np.uint32), D2.view(np.uint32))


@pytest.mark.parametrize("fmt", FP8s)
def test_fp8_inputs_match_the_per_element_oracle(fmt):
    """fp8 products are short dyadic numbers: sums of a few hundred of them
    are exact in fp64 in any order, so the two forms agree bit for bit."""
    rng = np.random.default_rng(fmt)
    M, N, K = 40, 24, 256
    dec = np.array([oracle.decode_fp8_e4m3(b) if fmt == oracle.FP8_E4M3
                    else oracle.decode_fp8_e5m2(b) for b in range(256)])
    finite = np.nonzero(np.isfinite(dec) & (np.abs(dec) <= 64))[0].astype(np.uint8)
    A = rng.choice(finite, size=(M, K))
    B = rng.choice(finite, size=(N, K))
    D1 = np.zeros(M * N, np.float32)
    D2 = np.zeros(M * N, np.float32)
    oracle.gemm(M, N, K, A.ravel(), K, ROW, B.ravel(), K, COL, None, N, D1, N, fmt, F32, F32, 0)
    oracle.gemm_product(M, N, K, A.ravel(), K, ROW, B.ravel(), K, COL, None, N, D2, N, fmt,
                        F32, F32, 0)
    assert np.array_equal(D1.view(np.uint32), D2.view(np.uint32))


@pytest.mark.parametrize("satf", [0, 1])
@pytest.mark.parametrize("layA,layB", [(ROW, COL), (COL, ROW)])
def test_int8_matches_gemm_i8(layA, layB, satf):
    rng = np.random.default_rng(11 + satf)
    M, N, K = 21, 30, 500
    A = rng.integers(-128, 128, size=(M, K) if layA == ROW else (K, M)).astype(np.int8)
    B = rng.integers(-128, 128, size=(K, N) if layB == ROW else (N, K)).astype(np.int8)
    lda, ldb = A.shape[1], B.shape[1]
    C = rng.integers(-2 ** 31, 2 ** 31, size=M * N, dtype=np.int64).astype(np.int32)
    D1 = np.zeros(M * N, np.int32)
    D2 = np.zeros(M * N, np.int32)
    oracle.gemm_i8(M, N, K, A.ravel(), lda, layA, B.ravel(), ldb, layB, C, N, ROW, D1, N, ROW, satf)
    oracle.gemm_i8_product(M, N, K, A.ravel(), lda, layA, B.ravel(), ldb, layB, C, N, ROW, D2, N,
                           ROW, satf)
    assert np.array_equal(D1, D2)


@pytest.mark.parametrize("satf", [0, 1])
def test_int8_long_sum_wraps_and_clamps(satf):
    """K = 140,000 products of 127 * 127: the sum 2,258,060,000 leaves the
    int32 range; it wraps to 2,258,060,000 - 2^32 or clamps to 2^31 - 1."""
    K = 140000
    A = np.full((1, K), 127, np.int8)
    B = np.full((K, 1), 127, np.int8)
    D = np.zeros(1, np.int32)
    oracle.gemm_i8_product(1, 1, K, A.ravel(), K, ROW, B.ravel(), 1, ROW, None, 1, ROW, D, 1,
                           ROW, satf)
    s = 127 * 127 * K
    assert int(D[0]) == (2 ** 31 - 1 if satf else s - 2 ** 32)


@pytest.mark.parametrize("out_dt", [F32, F16, BF16])
def test_satf_special_values(out_dt):
    """C = +Inf, -Inf, NaN with finite sums -> +MAX, -MAX, +0 under satf."""
    M, N, K = 3, 4, 2
    A = np.full(M * K, 0x3C00, np.uint16)            # 1.0
    B = np.full(K * N, 0x3C00, np.uint16)
    specials = np.array([np.inf, -np.inf, np.nan], np.float32)
    cv = np.repeat(specials, N).reshape(M, N)
    if out_dt == F32:
        C = cv.ravel().copy()
    elif out_dt == F16:
        C = cv.astype(np.float16).view(np.uint16).ravel().copy()
    else:
        C = (cv.view(np.uint32) >> 16).astype(np.uint16).ravel()
    D = np.zeros_like(C)
    acc = F16 if out_dt == F16 else F32
    oracle.gemm_product(M, N, K, A, K, ROW, B, N, ROW, C, N, D, N, F16, acc, out_dt, 1)
    Db = _bits_of(D, out_dt).reshape(M, N)
    mx = {F32: 0x7F7FFFFF, F16: 0x7BFF, BF16: 0x7F7F}[out_dt]
    sign = 0x80000000 if out_dt == F32 else 0x8000
    assert np.all(Db[0] == mx) and np.all(Db[1] == (sign | mx)) and np.all(Db[2] == 0)


def test_rejects_short_buffers_and_unknown_dtypes():
    A = np.zeros(10, np.uint16)
    with pytest.raises(ValueError):
        oracle.gemm_product(4, 4, 4, A, 4, ROW, np.zeros(16, np.uint16), 4, ROW, None, 4,
                            np.zeros(16, np.float32), 4, F16, F32, F32, 0)
    with pytest.raises(ValueError):
        oracle.decode_array(np.zeros(4, np.uint16), 99)
