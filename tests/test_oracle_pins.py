"""Pins of the CPU oracle against what the pages and the mathematics fix.

No GPU.  Each test checks the oracle against something other than itself:
numpy/torch conversions, exact rational arithmetic, integer closed forms,
the pages' worked 2x3 example, and invariants (in place, satf, padding).
"""
import itertools
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from exact_rne import (BF16, F16, F32, max_norm_bits, rne_bits, satf_bits,
                       value_of_bits16, value_of_out)

ROW, COL = oracle.ROW_MAJOR, oracle.COL_MAJOR
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


@pytest.fixture(scope="module", autouse=True)
def _built():
    oracle.build(force=False)


# --------------------------------------------------------------- decoding

def test_decode_f16_exhaustive_matches_numpy():
    lib = oracle._load()
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = np.array([lib.oracle_decode_f16(int(b)) for b in bits])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


def test_decode_bf16_exhaustive_matches_torch():
    lib = oracle._load()
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).double().numpy()
    got = np.array([lib.oracle_decode_bf16(int(b)) for b in bits])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


# --------------------------------------------------------------- rounding

def _round_probe_values(rng):
    """Random doubles over the fp16/bf16/fp32 ranges plus ties and thresholds."""
    vals = list(rng.standard_normal(3000) * np.exp2(rng.integers(-30, 20, 3000)))
    vals += list(rng.random(500) * 2 ** -14)       # fp16 subnormal range
    # exact ties between adjacent fp16 numbers, both parities
    for m in range(1024, 2048, 37):
        for e in (-24, -14, -3, 0, 5, 15):
            vals.append((m + 0.5) * 2.0 ** (e - 10))
            vals.append(-(m + 0.5) * 2.0 ** (e - 10))
    vals += [0.0, -0.0, 65504.0, 65519.99, 65520.0, 65535.0, 65536.0, 1e6, -65520.0,
             2.0 ** -24, 2.0 ** -25, 2.0 ** -25 * 1.0000001, 3 * 2.0 ** -26, 2.0 ** -14,
             float("inf"), float("-inf"), 1e300, -1e-300, 5e-324]
    return np.array(vals, dtype=np.float64)


def test_round_f16_matches_numpy():
    lib = oracle._load()
    vals = _round_probe_values(np.random.default_rng(7))
    with np.errstate(over="ignore"):
        ref = vals.astype(np.float16).view(np.uint16)
    got = np.array([lib.oracle_round_f16(float(v)) for v in vals], dtype=np.uint16)
    assert np.array_equal(got, ref), vals[got != ref][:10]
    # the overflow threshold of round-to-nearest-even into fp16
    assert lib.oracle_round_f16(65519.99) == 0x7BFF
    assert lib.oracle_round_f16(65520.0) == 0x7C00
    assert lib.oracle_round_f16(-65520.0) == 0xFC00
    assert lib.oracle_round_f16(float("nan")) & 0x7C00 == 0x7C00
    assert lib.oracle_round_f16(float("nan")) & 0x03FF != 0


def test_round_f32_matches_numpy():
    lib = oracle._load()
    rng = np.random.default_rng(8)
    vals = list(rng.standard_normal(5000) * np.exp2(rng.integers(-140, 120, 5000)))
    # exact fp32 ties (24-bit significand + half)
    for m in range(2 ** 23, 2 ** 24, 2 ** 23 // 97):
        vals.append((m + 0.5) * 2.0 ** -23)
    vals += [3.4028235677973366e38, 3.4028235677973366e38 * (1 + 2 ** -25), 3.5e38,
             2.0 ** -149, 2.0 ** -150, 1.5 * 2.0 ** -149, 2.0 ** -126]
    vals = np.array(vals, dtype=np.float64)
    with np.errstate(over="ignore"):
        ref = vals.astype(np.float32).view(np.uint32)
    got = np.array([lib.oracle_round_f32_bits(float(v)) for v in vals], dtype=np.uint32)
    assert np.array_equal(got, ref), vals[got != ref][:10]


def test_round_bf16_matches_torch_on_fp32_values_and_exact_rne_elsewhere():
    lib = oracle._load()
    rng = np.random.default_rng(9)
    # fp32-representable values: torch's fp32 -> bf16 cast is a single RNE step
    v32 = (rng.standard_normal(5000) * np.exp2(rng.integers(-135, 125, 5000))).astype(np.float32)
    ties = np.array([(m + 0.5) * 2.0 ** -7 for m in range(128, 256, 3)], dtype=np.float32)
    v32 = np.concatenate([v32, ties, -ties, np.array([3.3895e38, 3.3961e38, 3.4e38],
                                                     dtype=np.float32)])
    ref = torch.from_numpy(v32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = np.array([lib.oracle_round_bf16(float(v)) for v in v32], dtype=np.uint16)
    assert np.array_equal(got, ref), v32[got != ref][:10]
    # doubles that are NOT fp32 values (a cast through fp32 would round twice)
    probes = [1.0 + 2.0 ** -8 + 2.0 ** -40, 1.0 + 2.0 ** -8 - 2.0 ** -40,
              1.0 + 3 * 2.0 ** -8 + 2.0 ** -50, 2.0 ** -133 * 0.75, 2.0 ** -133 * 0.5]
    for x in probes:
        assert lib.oracle_round_bf16(x) == rne_bits(Fraction(x), BF16), x


def test_round_encoders_match_exact_rational_rne():
    lib = oracle._load()
    rng = np.random.default_rng(10)
    vals = rng.standard_normal(800) * np.exp2(rng.integers(-150, 130, 800))
    for x in vals:
        fx = Fraction(float(x))
        assert lib.oracle_round_f16(float(x)) == rne_bits(fx, F16)
        assert lib.oracle_round_bf16(float(x)) == rne_bits(fx, BF16)
        assert lib.oracle_round_f32_bits(float(x)) == rne_bits(fx, F32)


# ------------------------------------------------ the pages' 2x3 example

def _golden(name):
    out = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            k, v = line.split(":", 1)
            out[k.strip()] = [int(t) for t in v.split()]
    return out


def _f16(vals):
    return np.array(vals, dtype=np.float16).view(np.uint16)


def test_rowcol_2x3_example_addressing():
    g = _golden("rowcol_2x3.txt")
    M, N = g["matrix_rows"][0], g["matrix_cols"][0]
    expect = np.array(g["row_major_memory"], dtype=np.float32)
    eye3 = _f16(np.eye(3).ravel())
    eye2 = _f16(np.eye(2).ravel())
    # the 2x3 matrix as A (M=2, K=3) in both layouts, times B = I3
    for layout, mem, ld in ((ROW, g["row_major_memory"], 3), (COL, g["col_major_memory"], 2)):
        D = np.full(M * N, -1, dtype=np.float32)
        oracle.gemm(M, N, 3, _f16(mem), ld, layout, eye3, 3, ROW, None, N, D, N,
                    F16, F32, F32, 0)
        assert np.array_equal(D, expect), (layout, D)
    # the 2x3 matrix as B (K=2, N=3) in both layouts, with A = I2
    for layout, mem, ld in ((ROW, g["row_major_memory"], 3), (COL, g["col_major_memory"], 2)):
        D = np.full(2 * 3, -1, dtype=np.float32)
        oracle.gemm(2, 3, 2, eye2, 2, ROW, _f16(mem), ld, layout, None, 3, D, 3,
                    F16, F32, F32, 0)
        assert np.array_equal(D, expect), (layout, D)
    # the logical matrix agrees with the printed orders
    logical = np.array(g["logical"]).reshape(M, N)
    assert list(logical.ravel()) == g["row_major_memory"]
    assert list(logical.T.ravel()) == g["col_major_memory"]


# ------------------------------------------------ brute force vs exact sums

def _grid_values(rng, shape, dtype):
    """k * 2^e, |k| <= 255, e in [-8, 8]: exact in fp16 and bf16; fp64 sums of
    a few products of these are exact, so the oracle must equal RNE(exact)."""
    k = rng.integers(-255, 256, size=shape).astype(np.float64)
    e = rng.integers(-8, 9, size=shape).astype(np.float64)
    v = k * np.exp2(e)
    if dtype == F16:
        return v.astype(np.float16).view(np.uint16)
    if dtype == BF16:
        # bf16 holds 8 significant bits: |k| <= 255 fits exactly
        return (v.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    return v.astype(np.float32)


def _buffers(rng, M, N, K, layA, layB, in_dt, pad):
    a_outer, a_inner = (M, K) if layA == ROW else (K, M)
    b_outer, b_inner = (K, N) if layB == ROW else (N, K)
    lda, ldb = a_inner + pad, b_inner + pad
    nan = 0x7E00 if in_dt == F16 else 0x7FC0
    A = np.full((a_outer, max(lda, 1)), nan, dtype=np.uint16)
    B = np.full((b_outer, max(ldb, 1)), nan, dtype=np.uint16)
    A[:, :a_inner] = _grid_values(rng, (a_outer, a_inner), in_dt)
    B[:, :b_inner] = _grid_values(rng, (b_outer, b_inner), in_dt)
    return A, max(lda, 1), B, max(ldb, 1)


def _exact_D(M, N, K, A, lda, layA, B, ldb, layB, C, ldc, in_dt, out_dt):
    Af, Bf = A.ravel(), B.ravel()
    res = {}
    for i in range(M):
        for j in range(N):
            s = Fraction(0)
            for k in range(K):
                a = Af[i * lda + k] if layA == ROW else Af[k * lda + i]
                b = Bf[k * ldb + j] if layB == ROW else Bf[j * ldb + k]
                s += Fraction(value_of_bits16(int(a), in_dt)) * Fraction(value_of_bits16(int(b), in_dt))
            if C is not None:
                s += Fraction(value_of_out(C.ravel()[i * ldc + j], out_dt))
            res[(i, j)] = s
    return res


def _bits_of(D, out_dt):
    return D.view(np.uint32) if out_dt == F32 else D


CASES = list(itertools.product(
    [(1, 1, 1), (2, 3, 4), (3, 2, 5), (4, 4, 3), (1, 5, 2), (5, 1, 6), (3, 3, 0)],
    [ROW, COL], [ROW, COL], [F16, BF16],
    [(F32, F32), (F32, F16), (F32, BF16), (F16, F16)],
    ["none", "sep", "inplace"], [0, 1]))


@pytest.mark.parametrize("shape,layA,layB,in_dt,accout,cmode,satf",
                         [c for i, c in enumerate(CASES) if i % 5 == 0])
def test_bruteforce_tiny_vs_exact_rational(shape, layA, layB, in_dt, accout, cmode, satf):
    M, N, K = shape
    acc_dt, out_dt = accout
    rng = np.random.default_rng(hash((shape, layA, layB, in_dt, accout, cmode, satf)) % 2 ** 32)
    pad = int(rng.integers(0, 3))
    A, lda, B, ldb = _buffers(rng, M, N, K, layA, layB, in_dt, pad)
    ldd = N + int(rng.integers(0, 3))
    sentinel = np.float32(-777.25) if out_dt == F32 else np.uint16(0x5A5A)
    D = np.full((M + 1) * ldd, sentinel, dtype=np.float32 if out_dt == F32 else np.uint16)
    C, ldc = None, N
    if cmode != "none":
        cvals = _grid_values(rng, (M, N), out_dt)
        if cmode == "sep":
            ldc = N + 1
            C = np.zeros(M * ldc, dtype=D.dtype)
            C.reshape(M, ldc)[:, :N] = cvals
        else:
            ldc = ldd
            D.reshape(M + 1, ldd)[:M, :N] = cvals
            C = D
    exact = _exact_D(M, N, K, A, lda, layA, B, ldb, layB, C, ldc, in_dt, out_dt)
    oracle.gemm(M, N, K, A.ravel(), lda, layA, B.ravel(), ldb, layB,
                None if C is None else C, ldc, D, ldd, in_dt, acc_dt, out_dt, satf)
    Db = _bits_of(D, out_dt).reshape(M + 1, ldd)
    for (i, j), s in exact.items():
        want = rne_bits(s, out_dt)
        if satf:
            want = satf_bits(want, out_dt)
        got = int(Db[i, j])
        if s == 0:  # +0 and -0 are the same value
            assert value_of_out(D.reshape(M + 1, ldd)[i, j], out_dt) == 0.0
        else:
            assert got == want, (i, j, float(s), hex(got), hex(want))
    # nothing outside [0,M) x [0,N) was written
    sbits = int(np.array([sentinel]).view(np.uint32 if out_dt == F32 else np.uint16)[0])
    assert np.all(Db[:M, N:] == sbits) and np.all(Db[M, :] == sbits)


def test_plausible_mistakes_are_caught_by_the_exact_reference():
    """A transposed operand, a dropped C, a flipped sign or a short k loop all
    change the result on a non-square random case, so the brute-force pin
    above would fail for each of them."""
    rng = np.random.default_rng(99)
    M, N, K = 3, 4, 5
    A, lda, B, ldb = _buffers(rng, M, N, K, ROW, ROW, F16, 0)
    C = _grid_values(rng, (M, N), F32).ravel()
    exact = _exact_D(M, N, K, A, lda, ROW, B, ldb, ROW, C, N, F16, F32)
    want = np.array([float(np.float32(float(exact[(i, j)]))) for i in range(M) for j in range(N)])

    def run(M_, N_, K_, A_, lda_, layA, B_, ldb_, layB, C_):
        D = np.zeros(M * N, dtype=np.float32)
        oracle.gemm(M_, N_, K_, A_.ravel(), lda_, layA, B_.ravel(), ldb_, layB, C_, N, D, N,
                    F16, F32, F32, 0)
        return D.astype(np.float64)

    good = run(M, N, K, A, lda, ROW, B, ldb, ROW, C)
    assert np.array_equal(good, want)
    # B read as col-major with the same buffer: a transposed-operand mistake
    assert not np.array_equal(run(M, N, K, A, lda, ROW, B, N, COL, C), want)
    # C dropped
    assert not np.array_equal(run(M, N, K, A, lda, ROW, B, ldb, ROW, None), want)
    # last k term dropped
    assert not np.array_equal(run(M, N, K - 1, A, lda, ROW, B, ldb, ROW, C), want)
    # sign error on A
    negA = (A ^ np.uint16(0x8000)).astype(np.uint16)
    assert not np.array_equal(run(M, N, K, negA, lda, ROW, B, ldb, ROW, C), want)


# ------------------------------------------------ integer closed form

@pytest.mark.parametrize("layA,layB,in_dt", [(ROW, ROW, F16), (ROW, COL, BF16),
                                             (COL, ROW, BF16), (COL, COL, F16)])
def test_integer_inputs_equal_integer_matmul(layA, layB, in_dt):
    rng = np.random.default_rng(11)
    M, N, K = 37, 29, 53
    Ai = rng.integers(-2, 3, size=(M, K))
    Bi = rng.integers(-2, 3, size=(K, N))
    Ci = rng.integers(-50, 51, size=(M, N))
    ref = Ai @ Bi + Ci  # exact integer arithmetic
    Amem = Ai if layA == ROW else Ai.T
    Bmem = Bi if layB == ROW else Bi.T

    def bits(x):
        x = np.ascontiguousarray(x, dtype=np.float32)
        if in_dt == F16:
            return x.astype(np.float16).view(np.uint16)
        return (x.view(np.uint32) >> 16).astype(np.uint16)

    D = np.zeros(M * N, dtype=np.float32)
    oracle.gemm(M, N, K, bits(Amem).ravel(), Amem.shape[1], layA, bits(Bmem).ravel(),
                Bmem.shape[1], layB, Ci.astype(np.float32).ravel(), N, D, N,
                in_dt, F32, F32, 0)
    assert np.array_equal(D.reshape(M, N), ref.astype(np.float32))


# ------------------------------------------------ in place and satf

def test_inplace_equals_out_of_place_with_a_copy_of_C():
    rng = np.random.default_rng(12)
    M, N, K = 17, 23, 31
    A = (rng.random((M, K), dtype=np.float32) * 2 - 1).astype(np.float16).view(np.uint16)
    B = (rng.random((K, N), dtype=np.float32) * 2 - 1).astype(np.float16).view(np.uint16)
    C = rng.standard_normal((M, N)).astype(np.float32)
    D_sep = np.zeros(M * N, dtype=np.float32)
    oracle.gemm(M, N, K, A.ravel(), K, ROW, B.ravel(), N, ROW, C.ravel().copy(), N, D_sep, N,
                F16, F32, F32, 0)
    D_in = C.ravel().copy()
    oracle.gemm(M, N, K, A.ravel(), K, ROW, B.ravel(), N, ROW, D_in, N, D_in, N,
                F16, F32, F32, 0)
    assert np.array_equal(D_in.view(np.uint32), D_sep.view(np.uint32))


@pytest.mark.parametrize("out_dt", [F32, F16, BF16])
def test_satf_special_values(out_dt):
    """C in {+Inf, -Inf, NaN, 1.5} with a finite A*B: satf maps the results to
    {+MAX_NORM, -MAX_NORM, +0, unchanged}; without satf they stay special."""
    M, N, K = 1, 4, 2
    A = _f16([1.0, 2.0])
    B = _f16([1.0, 1.0, 1.0, -1.0, 0.5, 0.5, 0.25, 0.25])  # row-major 2x4
    if out_dt == F32:
        C = np.array([np.inf, -np.inf, np.nan, 1.5], dtype=np.float32)
    elif out_dt == F16:
        C = np.array([np.inf, -np.inf, np.nan, 1.5], dtype=np.float16).view(np.uint16)
    else:
        C = (np.array([np.inf, -np.inf, np.nan, 1.5], dtype=np.float32).view(np.uint32)
             >> 16).astype(np.uint16)
    acc = F16 if out_dt == F16 else F32
    for satf in (0, 1):
        D = np.zeros(4, dtype=C.dtype)
        oracle.gemm(M, N, K, A, K, ROW, B, N, ROW, C, N, D, N, F16, acc, out_dt, satf)
        vals = [value_of_out(x, out_dt) for x in D]
        mx = value_of_out(max_norm_bits(out_dt) if out_dt != F32 else
                          np.array([max_norm_bits(F32)], dtype=np.uint32).view(np.float32)[0],
                          out_dt)
        # A*B row = [1*1+2*0.5, 1*1+2*0.5, 1*1+2*0.25, -1+2*0.25] = [2, 2, 1.5, -0.5]
        if satf:
            assert vals[0] == mx and vals[1] == -mx
            assert vals[2] == 0.0 and not math.copysign(1.0, vals[2]) < 0
            assert vals[3] == 1.0
        else:
            assert vals[0] == math.inf and vals[1] == -math.inf and math.isnan(vals[2])
            assert vals[3] == 1.0


def test_fp16_overflow_threshold_and_satf():
    """Integer sums at and just below the fp16 round-to-Inf threshold 65520."""
    A = _f16([1008.0, 1.0])                                   # 1 x 2
    B = _f16([65.0, 64.0, 65.0, 0.0, 992.0, -1.0])            # 2 x 3 row-major
    # D = [1008*65, 1008*64 + 992, 1008*65 - 1] = [65520, 65504, 65519]
    for satf, want in ((0, [0x7C00, 0x7BFF, 0x7BFF]), (1, [0x7BFF, 0x7BFF, 0x7BFF])):
        D = np.zeros(3, dtype=np.uint16)
        oracle.gemm(1, 3, 2, A, 2, ROW, B, 3, ROW, None, 3, D, 3, F16, F16, F16, satf)
        assert [int(x) for x in D] == want, (satf, [hex(int(x)) for x in D])


def test_padding_and_rows_beyond_M_untouched():
    rng = np.random.default_rng(13)
    M, N, K, ldd = 5, 6, 7, 9
    A = (rng.random((M, K), dtype=np.float32)).astype(np.float16).view(np.uint16)
    B = (rng.random((K, N), dtype=np.float32)).astype(np.float16).view(np.uint16)
    D = np.full((M + 2) * ldd, 0x5A5A, dtype=np.uint16)
    oracle.gemm(M, N, K, A.ravel(), K, ROW, B.ravel(), N, ROW, None, N, D, ldd, F16, F32, F16, 0)
    Dm = D.reshape(M + 2, ldd)
    assert np.all(Dm[:M, N:] == 0x5A5A) and np.all(Dm[M:, :] == 0x5A5A)
    assert not np.any(Dm[:M, :N] == 0x5A5A)


def test_sampled_equals_full():
    rng = np.random.default_rng(14)
    M, N, K = 33, 47, 65
    A = (rng.random((K, M), dtype=np.float32) * 2 - 1).astype(np.float16).view(np.uint16)
    B = (rng.random((N, K), dtype=np.float32) * 2 - 1).astype(np.float16).view(np.uint16)
    C = rng.standard_normal((M, N)).astype(np.float32)
    D = np.zeros(M * N, dtype=np.float32)
    oracle.gemm(M, N, K, A.ravel(), M, COL, B.ravel(), K, COL, C.ravel(), N, D, N,
                F16, F32, F32, 0)
    rows = rng.integers(0, M, 200)
    cols = rng.integers(0, N, 200)
    S = oracle.gemm_sampled(M, N, K, A.ravel(), M, COL, B.ravel(), K, COL, C.ravel(), N,
                            rows, cols, F16, F32, F32, 0)
    assert np.array_equal(S, D.reshape(M, N)[rows, cols])


def test_random_fp16_within_half_ulp_of_exact():
    """Unrestricted U[-1,1] fp16 inputs (fp64 sums may round): the oracle's
    output is within half an fp32 ulp of the exact value plus the fp64
    accumulation error bound K * 2^-53 * sum|a*b|."""
    rng = np.random.default_rng(15)
    M, N, K = 4, 5, 64
    A = (rng.random((M, K), dtype=np.float32) * 2 - 1).astype(np.float16)
    B = (rng.random((K, N), dtype=np.float32) * 2 - 1).astype(np.float16)
    D = np.zeros(M * N, dtype=np.float32)
    oracle.gemm(M, N, K, A.view(np.uint16).ravel(), K, ROW, B.view(np.uint16).ravel(), N, ROW,
                None, N, D, N, F16, F32, F32, 0)
    for i in range(M):
        for j in range(N):
            terms = [Fraction(float(A[i, k])) * Fraction(float(B[k, j])) for k in range(K)]
            s = sum(terms, Fraction(0))
            absum = float(sum(abs(t) for t in terms))
            got = Fraction(float(D[i * N + j]))
            ulp = float(np.spacing(np.float32(abs(float(s))))) if s != 0 else 2.0 ** -149
            bound = Fraction(ulp) / 2 + Fraction(K * 2.0 ** -53 * absum)
            assert abs(got - s) <= bound
