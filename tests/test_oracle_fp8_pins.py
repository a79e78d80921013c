"""Pins of the oracle's OCP fp8 inputs (E4M3, E5M2).

No GPU.  The decoders are checked exhaustively against torch's own
float8_e4m3fn / float8_e5m2 conversions (an independent implementation of the
same OCP formats) and against the formats' published extreme values; small
GEMMs on fp8 inputs against exact rational sums rounded by the hand-written
round-half-to-even of exact_rne.
"""
import itertools
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from exact_rne import BF16, F16, F32, rne_bits, satf_bits, value_of_out

ROW, COL = oracle.ROW_MAJOR, oracle.COL_MAJOR
E4M3, E5M2 = oracle.FP8_E4M3, oracle.FP8_E5M2


@pytest.fixture(scope="module", autouse=True)
def _built():
    oracle.build(force=False)


def _torch_decode(fmt):
    dt = torch.float8_e4m3fn if fmt == E4M3 else torch.float8_e5m2
    return torch.arange(256, dtype=torch.int32).to(torch.uint8).view(dt).to(torch.float64).numpy()


@pytest.mark.parametrize("fmt", [E4M3, E5M2])
def test_decode_exhaustive_matches_torch(fmt):
    dec = oracle.decode_fp8_e4m3 if fmt == E4M3 else oracle.decode_fp8_e5m2
    ours = np.array([dec(b) for b in range(256)])
    ref = _torch_decode(fmt)
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(ours[ok], ref[ok])


def test_published_extreme_values():
    d4, d5 = oracle.decode_fp8_e4m3, oracle.decode_fp8_e5m2
    assert d4(0x7E) == 448.0 and d4(0xFE) == -448.0          # largest finite E4M3
    assert d4(0x08) == 2.0 ** -6 and d4(0x01) == 2.0 ** -9   # smallest normal, subnormal
    assert np.isnan(d4(0x7F)) and np.isnan(d4(0xFF))         # the only NaNs, no Inf
    assert d4(0x38) == 1.0 and d4(0x00) == 0.0 and d4(0x80) == 0.0
    assert d5(0x7B) == 57344.0 and d5(0x7C) == np.inf and d5(0xFC) == -np.inf
    assert d5(0x04) == 2.0 ** -14 and d5(0x01) == 2.0 ** -16
    assert all(np.isnan(d5(b)) for b in (0x7D, 0x7E, 0x7F, 0xFD))
    assert d5(0x3C) == 1.0


def _finite_bytes(rng, shape, fmt):
    x = rng.integers(0, 256, size=shape).astype(np.uint8)
    if fmt == E4M3:
        return np.where((x & 0x7F) == 0x7F, x & 0xF7, x).astype(np.uint8)
    return np.where(((x >> 2) & 0x1F) == 0x1F, x & 0xBF, x).astype(np.uint8)


CASES = list(itertools.product([(1, 1, 1), (2, 3, 5), (3, 2, 7), (4, 4, 0)], [ROW, COL],
                               [ROW, COL], [E4M3, E5M2], [F32, F16, BF16], [0, 1]))


@pytest.mark.parametrize("shape,la,lb,fmt,out_dt,satf", [c for n, c in enumerate(CASES)
                                                        if n % 3 == 0])
def test_bruteforce_fp8_vs_exact_rational(shape, la, lb, fmt, out_dt, satf):
    M, N, K = shape
    rng = np.random.default_rng(hash((shape, la, lb, fmt, out_dt, satf)) % 2 ** 32)
    a_outer, a_inner = (M, K) if la == ROW else (K, M)
    b_outer, b_inner = (K, N) if lb == ROW else (N, K)
    lda, ldb = max(1, a_inner) + 1, max(1, b_inner) + 2
    A = _finite_bytes(rng, a_outer * lda, fmt)
    B = _finite_bytes(rng, b_outer * ldb, fmt)
    odt = np.float32 if out_dt == F32 else np.uint16
    C = np.zeros(M * N, dtype=odt)
    cv = rng.integers(-50, 51, size=M * N).astype(np.float32) * np.float32(0.25)
    C[:] = cv if out_dt == F32 else (cv.astype(np.float16).view(np.uint16) if out_dt == F16
                                      else (cv.view(np.uint32) >> 16).astype(np.uint16))
    D = np.zeros(M * N, dtype=odt)
    acc = F16 if (out_dt == F16 and satf) else F32
    oracle.gemm(M, N, K, A, lda, la, B, ldb, lb, C, N, D, N, fmt, acc, out_dt, satf)
    dec = oracle.decode_fp8_e4m3 if fmt == E4M3 else oracle.decode_fp8_e5m2
    tdec = _torch_decode(fmt)  # exact values, independent decoder
    for i in range(M):
        for j in range(N):
            s = Fraction(0)
            for k in range(K):
                a = A[i * lda + k] if la == ROW else A[k * lda + i]
                b = B[k * ldb + j] if lb == ROW else B[j * ldb + k]
                s += Fraction(float(tdec[a])) * Fraction(float(tdec[b]))
            s += Fraction(value_of_out(C[i * N + j], out_dt))
            want = rne_bits(s, out_dt)
            if satf:
                want = satf_bits(want, out_dt)
            got = D[i * N + j]
            gb = int(np.array(got).view(np.uint32)) if out_dt == F32 else int(got)
            if s == 0:
                assert value_of_out(got, out_dt) == 0.0
            else:
                assert gb == want, (i, j, float(s), hex(gb), hex(want))
    assert dec(0x38 if fmt == E4M3 else 0x3C) == 1.0


@pytest.mark.parametrize("fmt", [E4M3, E5M2])
def test_fp8_through_the_extended_oracle(fmt):
    """gemm_ex with default epilogue equals gemm for fp8 inputs, and a
    column-major D is the transpose."""
    rng = np.random.default_rng(9)
    M, N, K = 6, 7, 64
    A = _finite_bytes(rng, M * K, fmt)
    B = _finite_bytes(rng, K * N, fmt)
    D1 = np.zeros(M * N, dtype=np.float32)
    D2 = np.zeros(M * N, dtype=np.float32)
    D3 = np.zeros(N * M, dtype=np.float32)
    oracle.gemm(M, N, K, A, K, ROW, B, N, ROW, None, N, D1, N, fmt, F32, F32, 0)
    oracle.gemm_ex(M, N, K, A, K, ROW, B, N, ROW, None, N, ROW, D2, N, ROW, fmt, F32, F32, 0)
    oracle.gemm_ex(M, N, K, A, K, ROW, B, N, ROW, None, M, ROW, D3, M, COL, fmt, F32, F32, 0)
    assert np.array_equal(D1.view(np.uint32), D2.view(np.uint32))
    assert np.array_equal(D1.reshape(M, N), D3.reshape(N, M).T)
