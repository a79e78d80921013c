"""Pins of the oracle's extended epilogue, D = act(alpha*(A x B) + beta*C + bias),
with row- or column-major C and D.

No GPU.  The checks are against things other than the oracle's own code:
exact rational arithmetic with a hand-written round-half-to-even, the
unextended (already pinned) oracle, the standard normal CDF from a Simpson
quadrature of its density and from printed table values, and the identities
GELU(x) - GELU(-x) = x and "a column-major D is the transpose of a row-major
one".
"""
import itertools
import math
from fractions import Fraction

import numpy as np
import pytest

import oracle
from exact_rne import BF16, F16, F32, rne_bits, satf_bits, value_of_bits16, value_of_out

ROW, COL = oracle.ROW_MAJOR, oracle.COL_MAJOR
NONE, RELU, GELU = oracle.ACT_NONE, oracle.ACT_RELU, oracle.ACT_GELU


@pytest.fixture(scope="module", autouse=True)
def _built():
    oracle.build(force=False)


# ------------------------------------------------ small exact-value grids

def _grid(rng, shape, dtype):
    """k * 2^e with |k| <= 63, e in [-4, 4]: exact in fp16, bf16 and fp32, and
    every sum formed below stays exact in fp64."""
    k = rng.integers(-63, 64, size=shape).astype(np.float64)
    e = rng.integers(-4, 5, size=shape).astype(np.float64)
    v = k * np.exp2(e)
    if dtype == F16:
        return v.astype(np.float16).view(np.uint16)
    if dtype == BF16:
        return (v.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    return v.astype(np.float32)


def _operands(rng, M, N, K, layA, layB, in_dt):
    a_outer, a_inner = (M, K) if layA == ROW else (K, M)
    b_outer, b_inner = (K, N) if layB == ROW else (N, K)
    A = _grid(rng, (a_outer, max(a_inner, 1)), in_dt)
    B = _grid(rng, (b_outer, max(b_inner, 1)), in_dt)
    return A, max(a_inner, 1), B, max(b_inner, 1)


def _exact_sum(M, N, K, A, lda, layA, B, ldb, layB, in_dt):
    """S(i,j) = sum_k A(i,k) B(k,j) as Fractions, addressed with the pages'
    row-major r*ld + c and column-major c*ld + r offsets."""
    Af, Bf = A.ravel(), B.ravel()
    S = {}
    for i in range(M):
        for j in range(N):
            s = Fraction(0)
            for k in range(K):
                a = Af[i * lda + k] if layA == ROW else Af[k * lda + i]
                b = Bf[k * ldb + j] if layB == ROW else Bf[j * ldb + k]
                s += Fraction(value_of_bits16(int(a), in_dt)) * \
                    Fraction(value_of_bits16(int(b), in_dt))
            S[(i, j)] = s
    return S


def _at(layout, ld, i, j):
    return i * ld + j if layout == ROW else j * ld + i


def _bits(x, out_dt):
    return int(np.asarray(x).view(np.uint32)) if out_dt == F32 else int(x)


# ------------------------------------------------ defaults = the base oracle

@pytest.mark.parametrize("out_dt,acc_dt", [(F32, F32), (F16, F16), (BF16, F32)])
@pytest.mark.parametrize("cmode", ["none", "sep", "inplace"])
def test_defaults_reproduce_the_unextended_oracle(out_dt, acc_dt, cmode):
    rng = np.random.default_rng(11 + out_dt + 7 * len(cmode))
    M, N, K = 7, 9, 33
    in_dt = F16 if acc_dt == F16 else BF16
    A = (rng.standard_normal((M, K)).astype(np.float32))
    B = (rng.standard_normal((K, N)).astype(np.float32))
    if in_dt == F16:
        A, B = A.astype(np.float16).view(np.uint16), B.astype(np.float16).view(np.uint16)
    else:
        A = (A.view(np.uint32) >> 16).astype(np.uint16)
        B = (B.view(np.uint32) >> 16).astype(np.uint16)
    odt = np.float32 if out_dt == F32 else np.uint16
    cvals = _grid(rng, (M * N,), out_dt)
    D1 = np.zeros(M * N, dtype=odt)
    D2 = np.zeros(M * N, dtype=odt)
    C1 = C2 = None
    if cmode == "sep":
        C1 = C2 = cvals
    elif cmode == "inplace":
        D1[:], D2[:] = cvals, cvals
        C1, C2 = D1, D2
    oracle.gemm(M, N, K, A.ravel(), K, ROW, B.ravel(), N, ROW, C1, N, D1, N,
                in_dt, acc_dt, out_dt, 0)
    oracle.gemm_ex(M, N, K, A.ravel(), K, ROW, B.ravel(), N, ROW, C2, N, ROW, D2, N, ROW,
                   in_dt, acc_dt, out_dt, 0)
    assert np.array_equal(D1.view(np.uint32 if out_dt == F32 else np.uint16),
                          D2.view(np.uint32 if out_dt == F32 else np.uint16))


# ------------------------------------------------ brute force, exact

ALPHAS = [1.0, -2.0, 0.5, 0.25, 0.0]
BETAS = [1.0, 0.5, -1.0, 0.0]
EX_CASES = list(itertools.product(
    [(1, 1, 1), (2, 3, 4), (3, 2, 5), (4, 4, 0)],
    [(ROW, ROW), (ROW, COL), (COL, ROW), (COL, COL)],   # (layoutC, layoutD)
    [NONE, RELU],
    [F32, F16, BF16],
    range(len(ALPHAS)),
    ["bias", "nobias"]))


@pytest.mark.parametrize("shape,cd,act,out_dt,ai,bias_mode",
                         [c for n, c in enumerate(EX_CASES) if n % 7 == 0])
def test_bruteforce_extended_vs_exact_rational(shape, cd, act, out_dt, ai, bias_mode):
    M, N, K = shape
    layC, layD = cd
    alpha = ALPHAS[ai]
    beta = BETAS[(ai + act) % len(BETAS)]
    seed = hash((shape, cd, act, out_dt, ai, bias_mode)) % 2 ** 32
    rng = np.random.default_rng(seed)
    layA, layB = ROW if seed % 2 else COL, COL if seed % 3 else ROW
    in_dt = BF16 if out_dt == BF16 else F16
    acc_dt = F16 if (out_dt == F16 and seed % 2) else F32
    A, lda, B, ldb = _operands(rng, M, N, K, layA, layB, in_dt)
    odt = np.float32 if out_dt == F32 else np.uint16
    ldc = (N if layC == ROW else M) + 1
    ldd = (N if layD == ROW else M) + 2
    outer_c = M if layC == ROW else N
    outer_d = M if layD == ROW else N
    C = np.zeros(outer_c * ldc, dtype=odt)
    cvals = _grid(rng, (M, N), out_dt)
    for i in range(M):
        for j in range(N):
            C[_at(layC, ldc, i, j)] = cvals[i, j]
    if beta == 0.0:  # beta == 0: C must not be read, so poison it
        C[:] = np.float32(np.nan) if out_dt == F32 else (0x7E00 if out_dt == F16 else 0x7FC0)
    bias = _grid(rng, (N,), F32) if bias_mode == "bias" else None
    sentinel = np.float32(-777.25) if out_dt == F32 else np.uint16(0x5A5A)
    D = np.full((outer_d + 1) * ldd, sentinel, dtype=odt)
    oracle.gemm_ex(M, N, K, A.ravel(), lda, layA, B.ravel(), ldb, layB, C, ldc, layC,
                   D, ldd, layD, in_dt, acc_dt, out_dt, 1, alpha, beta, bias, act)

    S = _exact_sum(M, N, K, A, lda, layA, B, ldb, layB, in_dt)
    written = set()
    for (i, j), s in S.items():
        v = Fraction(alpha) * s
        if beta != 0.0:
            v += Fraction(beta) * Fraction(value_of_out(C[_at(layC, ldc, i, j)], out_dt))
        if bias is not None:
            v += Fraction(float(bias[j]))
        if act == RELU:
            v = max(v, Fraction(0))
        want = satf_bits(rne_bits(v, out_dt), out_dt)
        off = _at(layD, ldd, i, j)
        written.add(off)
        got = D[off]
        if v == 0:
            assert value_of_out(got, out_dt) == 0.0, (i, j)
            if act == RELU:  # ReLU gives +0, never -0
                assert _bits(got, out_dt) == 0, (i, j)
        else:
            assert _bits(got, out_dt) == want, (i, j, float(v), hex(_bits(got, out_dt)), hex(want))
    sbits = _bits(sentinel, out_dt)
    untouched = [o for o in range(D.size) if o not in written]
    assert all(_bits(D[o], out_dt) == sbits for o in untouched)


def test_plausible_epilogue_mistakes_change_the_exact_result():
    """Bias added per row instead of per column, alpha applied to C as well,
    beta dropped, or ReLU applied before the bias each change the exact
    result of this non-square case, so the brute force above would catch
    them in the oracle."""
    rng = np.random.default_rng(5)
    M, N, K = 2, 3, 4
    A, lda, B, ldb = _operands(rng, M, N, K, ROW, ROW, F16)
    S = _exact_sum(M, N, K, A, lda, ROW, B, ldb, ROW, F16)
    C = _grid(rng, (M, N), F32)
    bias = np.array([3.0, -5.0, 0.75], dtype=np.float32)
    alpha, beta = Fraction(-2), Fraction(1, 2)

    def result(f):
        return [f(i, j, S[(i, j)]) for i in range(M) for j in range(N)]

    relu = lambda v: max(v, Fraction(0))
    good = result(lambda i, j, s: relu(alpha * s + beta * Fraction(float(C[i, j])) + Fraction(float(bias[j]))))
    D = np.zeros(M * N, dtype=np.float32)
    oracle.gemm_ex(M, N, K, A.ravel(), lda, ROW, B.ravel(), ldb, ROW, C.ravel(), N, ROW,
                   D, N, ROW, F16, F32, F32, 0, -2.0, 0.5, bias, RELU)
    assert [float(x) for x in D] == [float(np.float32(float(v))) for v in good]
    mistakes = [
        lambda i, j, s: relu(alpha * s + beta * Fraction(float(C[i, j])) + Fraction(float(bias[i]))),
        lambda i, j, s: relu(alpha * (s + beta * Fraction(float(C[i, j]))) + Fraction(float(bias[j]))),
        lambda i, j, s: relu(alpha * s + Fraction(float(C[i, j])) + Fraction(float(bias[j]))),
        lambda i, j, s: relu(alpha * s + beta * Fraction(float(C[i, j]))) + Fraction(float(bias[j])),
    ]
    for bad in mistakes:
        assert result(bad) != good


# ------------------------------------------------ activations

def _phi_simpson(x: float, n: int = 20000) -> float:
    """Standard normal CDF: 1/2 + integral_0^x of exp(-t^2/2)/sqrt(2 pi) dt,
    composite Simpson rule (needs only math.exp)."""
    if x == 0.0:
        return 0.5
    h = x / n
    acc = 0.0
    for m in range(n + 1):
        w = 1 if m in (0, n) else (4 if m % 2 else 2)
        t = m * h
        acc += w * math.exp(-0.5 * t * t)
    return 0.5 + acc * h / 3.0 / math.sqrt(2.0 * math.pi)


# Printed table values of the standard normal CDF.
PHI_TABLE = {0.5: 0.6914624612740131, 1.0: 0.8413447460685429,
             2.0: 0.9772498680518208, 3.0: 0.9986501019683699,
             -1.0: 0.15865525393145707}


def test_gelu_matches_x_times_normal_cdf():
    for x, phi in PHI_TABLE.items():
        assert math.isclose(oracle.activation(x, GELU), x * phi, rel_tol=1e-13), x
    for x in np.linspace(-6.0, 6.0, 49):
        x = float(x)
        # for x << 0 both sides form 1 + erf (resp. 1/2 - integral) by
        # cancellation, and the quadrature's own error is about 1e-15, so
        # the absolute accuracy left is about |x| * 1e-14
        assert math.isclose(oracle.activation(x, GELU), x * _phi_simpson(x),
                            rel_tol=1e-11, abs_tol=1e-14 * max(1.0, abs(x))), x


def test_gelu_identities_and_limits():
    rng = np.random.default_rng(3)
    for x in rng.standard_normal(200) * 4:
        x = float(x)
        g, gm = oracle.activation(x, GELU), oracle.activation(-x, GELU)
        assert math.isclose(g - gm, x, rel_tol=1e-14, abs_tol=1e-15), x  # x*Phi(x) + x*Phi(-x) = x
    assert oracle.activation(0.0, GELU) == 0.0
    assert oracle.activation(math.inf, GELU) == math.inf
    assert oracle.activation(-math.inf, GELU) == 0.0
    assert math.isnan(oracle.activation(math.nan, GELU))
    assert 0.0 > oracle.activation(-40.0, GELU) > -1e-300 or oracle.activation(-40.0, GELU) == 0.0


def test_relu_and_identity():
    for x in (-3.5, -1e-300, 0.0, 2.25, 1e300):
        assert oracle.activation(x, RELU) == (x if x > 0 else 0.0)
        assert oracle.activation(x, NONE) == x
    assert math.copysign(1.0, oracle.activation(-0.0, RELU)) == 1.0
    assert math.isnan(oracle.activation(math.nan, RELU))
    assert oracle.activation(math.inf, RELU) == math.inf
    assert oracle.activation(-math.inf, RELU) == 0.0


def test_gelu_gemm_element_rounds_the_exact_gelu():
    """1 x N x K GEMM with GELU, fp32 out: each output is the fp32 rounding of
    s * Phi(s), s = alpha * S with S exact (Fractions) and Phi from the
    quadrature; alpha (a power of two) puts s into [-4, 4]."""
    rng = np.random.default_rng(8)
    M, N, K = 1, 32, 6
    A, lda, B, ldb = _operands(rng, M, N, K, ROW, ROW, F16)
    S = _exact_sum(M, N, K, A, lda, ROW, B, ldb, ROW, F16)
    smax = max(abs(float(v)) for v in S.values())
    alpha = 2.0 ** -math.ceil(math.log2(smax / 4.0))
    D = np.zeros(N, dtype=np.float32)
    oracle.gemm_ex(M, N, K, A.ravel(), lda, ROW, B.ravel(), ldb, ROW, None, N, ROW,
                   D, N, ROW, F16, F32, F32, 0, alpha, 0.0, None, GELU)
    curved = 0
    for j in range(N):
        s = float(Fraction(alpha) * S[(0, j)])
        want = s * _phi_simpson(s)
        curved += 0.1 < abs(s) < 3.0
        tol = float(np.spacing(np.float32(abs(want)))) + 1e-14 * abs(s)
        assert abs(float(D[j]) - want) <= tol, (j, s, float(D[j]), want)
    assert curved >= 8  # enough outputs away from GELU's linear tails


# ------------------------------------------------ layouts, sampling

@pytest.mark.parametrize("out_dt", [F32, F16])
def test_column_major_d_is_the_transpose(out_dt):
    rng = np.random.default_rng(21)
    M, N, K = 5, 7, 19
    A, lda, B, ldb = _operands(rng, M, N, K, ROW, COL, F16)
    odt = np.float32 if out_dt == F32 else np.uint16
    C = _grid(rng, (M, N), out_dt)
    CT = np.ascontiguousarray(C.T)
    bias = _grid(rng, (N,), F32)
    Dr = np.zeros(M * N, dtype=odt)
    Dc = np.zeros(N * M, dtype=odt)
    args = (F16, F32 if out_dt == F32 else F16, out_dt, 0, 0.5, -1.0, bias, GELU)
    oracle.gemm_ex(M, N, K, A.ravel(), lda, ROW, B.ravel(), ldb, COL, C.ravel(), N, ROW,
                   Dr, N, ROW, *args)
    oracle.gemm_ex(M, N, K, A.ravel(), lda, ROW, B.ravel(), ldb, COL, CT.ravel(), M, COL,
                   Dc, M, COL, *args)
    assert np.array_equal(Dr.reshape(M, N), Dc.reshape(N, M).T)


def test_in_place_column_major():
    rng = np.random.default_rng(22)
    M, N, K = 4, 6, 9
    A, lda, B, ldb = _operands(rng, M, N, K, COL, ROW, F16)
    C = _grid(rng, (N * M,), F32)
    D = C.copy()
    ref = np.zeros_like(C)
    oracle.gemm_ex(M, N, K, A.ravel(), lda, COL, B.ravel(), ldb, ROW, C, M, COL, ref, M, COL,
                   F16, F32, F32, 0, -0.5, 2.0, None, RELU)
    oracle.gemm_ex(M, N, K, A.ravel(), lda, COL, B.ravel(), ldb, ROW, D, M, COL, D, M, COL,
                   F16, F32, F32, 0, -0.5, 2.0, None, RELU)
    assert np.array_equal(D, ref)


def test_sampled_extended_equals_full():
    rng = np.random.default_rng(23)
    M, N, K = 9, 11, 40
    A, lda, B, ldb = _operands(rng, M, N, K, ROW, ROW, BF16)
    C = _grid(rng, (M * N,), BF16)
    bias = _grid(rng, (N,), F32)
    D = np.zeros(M * N, dtype=np.uint16)
    oracle.gemm_ex(M, N, K, A.ravel(), lda, ROW, B.ravel(), ldb, ROW, C, N, ROW, D, N, ROW,
                   BF16, F32, BF16, 1, 0.75, -0.5, bias, GELU)
    rows = rng.integers(0, M, 30)
    cols = rng.integers(0, N, 30)
    got = oracle.gemm_ex_sampled(M, N, K, A.ravel(), lda, ROW, B.ravel(), ldb, ROW, C, N, ROW,
                                 rows, cols, BF16, F32, BF16, 1, 0.75, -0.5, bias, GELU)
    assert np.array_equal(got, D.reshape(M, N)[rows, cols])


def test_rejects_unknown_activation_and_layout():
    A = np.zeros(4, dtype=np.uint16)
    D = np.zeros(4, dtype=np.float32)
    with pytest.raises(ValueError):
        oracle.gemm_ex(2, 2, 2, A, 2, ROW, A, 2, ROW, None, 2, ROW, D, 2, ROW,
                       F16, F32, F32, 0, 1.0, 1.0, None, 7)
    with pytest.raises(ValueError):
        oracle.gemm_ex(2, 2, 2, A, 2, ROW, A, 2, ROW, None, 2, ROW, D, 2, 5,
                       F16, F32, F32, 0, 1.0, 1.0, None, NONE)
