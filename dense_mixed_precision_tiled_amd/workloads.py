"""Seeded synthetic inputs for D = A x B + C.

This module only draws random numbers and lays them out in memory; it holds
none of the multiply-accumulate arithmetic.  Both the GPU path (tests, bench,
smoke) and the CPU oracle consume what it produces.

Storage conventions (the call contract of ``gemm_run``):

* A is M x K.  Row-major: ``A(i,k) = A[i*lda + k]``, buffer shape (M, lda).
  Col-major: ``A(i,k) = A[k*lda + i]``, buffer shape (K, lda).
* B is K x N.  Row-major: ``B(k,j) = B[k*ldb + j]``, buffer shape (K, ldb).
  Col-major: ``B(k,j) = B[j*ldb + k]``, buffer shape (N, ldb).
* C and D are row-major M x N with ldc / ldd, buffer shape (M, ld).

A and B hold 16-bit patterns (uint16) of fp16 or bf16; C and D hold float32
or 16-bit patterns of the output dtype.  Padding columns of A and B (between
the used extent and ld) are filled with NaN patterns, and D's padding with a
sentinel, so a kernel that reads or writes outside the matrices shows up.

Value recipes (the pages measure on synthetic square matrices only):
``uniform``: U[-1,1) drawn in fp32, rounded to the input dtype (RNE);
``normal``: N(0,1) drawn in fp32, rounded to the input dtype;
``int``: integers in {-2,...,2} (exact in fp16/bf16).
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np
import torch

F32, F16, BF16 = 0, 1, 2
FP8_E4M3, FP8_E5M2 = 5, 6
ROW_MAJOR, COL_MAJOR = 0, 1

NAN16 = {F16: 0x7E00, BF16: 0x7FC0}
NAN8 = {FP8_E4M3: 0x7F, FP8_E5M2: 0x7E}
SENTINEL_F32 = np.float32(-12345.5)
SENTINEL_16 = np.uint16(0x5A5A)


def to_bits8(x: np.ndarray, dtype: int) -> np.ndarray:
    """Round float32 values to OCP fp8 (E4M3 or E5M2, torch's conversion) -> uint8 bits."""
    dt = torch.float8_e4m3fn if dtype == FP8_E4M3 else torch.float8_e5m2
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(dt)
    return t.view(torch.uint8).numpy()


def to_bits16(x: np.ndarray, dtype: int) -> np.ndarray:
    """Round float32 values to fp16/bf16 (round-to-nearest-even) -> uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    if dtype == F16:
        return x.astype(np.float16).view(np.uint16)
    if dtype == BF16:
        t = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16)
        return t.numpy().view(np.uint16)
    raise ValueError("16-bit dtype expected")


def from_bits16(b: np.ndarray, dtype: int) -> np.ndarray:
    """uint16 patterns -> float32 values (exact)."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    if dtype == F16:
        return b.view(np.float16).astype(np.float32)
    if dtype == BF16:
        return (b.astype(np.uint32) << 16).view(np.float32)
    raise ValueError("16-bit dtype expected")


def _draw(rng: np.random.Generator, shape, values: str) -> np.ndarray:
    if values == "uniform":
        return rng.random(shape, dtype=np.float32) * np.float32(2.0) - np.float32(1.0)
    if values == "normal":
        return rng.standard_normal(shape, dtype=np.float32)
    if values == "int":
        return rng.integers(-2, 3, size=shape).astype(np.float32)
    if values == "zero":
        return np.zeros(shape, dtype=np.float32)
    raise ValueError(values)


@dataclasses.dataclass
class Problem:
    """One call's worth of host-side inputs, in the gemm_run argument order."""
    name: str
    M: int
    N: int
    K: int
    A: np.ndarray          # 2-D uint16 buffer (outer, lda)
    lda: int
    layoutA: int
    B: np.ndarray          # 2-D uint16 buffer (outer, ldb)
    ldb: int
    layoutB: int
    C: Optional[np.ndarray]  # 2-D buffer (M, ldc) or None
    ldc: int
    D: np.ndarray          # 2-D buffer (M, ldd), initialised to the sentinel (or = C)
    ldd: int
    in_dtype: int
    acc_dtype: int
    out_dtype: int
    satf: int
    inplace: bool = False  # C and D are the same buffer
    extra: dict = dataclasses.field(default_factory=dict)  # recipe details (e.g. scaled rows)

    @property
    def flops(self) -> int:
        return 2 * self.M * self.N * self.K


def _operand(rng, rows: int, cols: int, ld: int, dtype: int, values: str) -> np.ndarray:
    """A (rows, ld) buffer of 16-bit (uint16) or fp8 (uint8) patterns whose
    first `cols` columns hold values, pad = NaN."""
    if dtype in NAN8:
        buf = np.full((rows, ld), NAN8[dtype], dtype=np.uint8)
        if rows and cols:
            buf[:, :cols] = to_bits8(_draw(rng, (rows, cols), values), dtype)
        return buf
    buf = np.full((rows, ld), NAN16[dtype], dtype=np.uint16)
    if rows and cols:
        buf[:, :cols] = to_bits16(_draw(rng, (rows, cols), values), dtype)
    return buf


def _out_buffer(M: int, ld: int, out_dtype: int) -> np.ndarray:
    if out_dtype == F32:
        return np.full((M, ld), SENTINEL_F32, dtype=np.float32)
    return np.full((M, ld), SENTINEL_16, dtype=np.uint16)


def _round_up(n: int, a: int) -> int:
    return (n + a - 1) // a * a


def make_problem(M: int, N: int, K: int, *, layoutA=ROW_MAJOR, layoutB=ROW_MAJOR,
                 in_dtype=F16, acc_dtype=F32, out_dtype=F32, satf=0,
                 values="uniform", c_values: Optional[str] = None, inplace=False,
                 lda=None, ldb=None, ldc=None, ldd=None, seed=1234,
                 name="custom", align=1) -> Problem:
    """Build a seeded problem.  c_values=None means C = NULL (C = 0).
    Unset lda / ldb are the operand's line length rounded up to a multiple
    of ``align`` elements (8: 16-byte lines for 16-bit inputs)."""
    rng_a = np.random.default_rng(seed)
    rng_b = np.random.default_rng(seed + 1)
    rng_c = np.random.default_rng(seed + 2)
    a_outer, a_inner = (M, K) if layoutA == ROW_MAJOR else (K, M)
    b_outer, b_inner = (K, N) if layoutB == ROW_MAJOR else (N, K)
    lda = _round_up(max(1, a_inner), align) if lda is None else lda
    ldb = _round_up(max(1, b_inner), align) if ldb is None else ldb
    ldd = max(1, N) if ldd is None else ldd
    A = _operand(rng_a, a_outer, a_inner, lda, in_dtype, values)
    B = _operand(rng_b, b_outer, b_inner, ldb, in_dtype, values)
    C = None
    if inplace:
        ldc = ldd
        D = _out_buffer(M, ldd, out_dtype)
        if c_values is None:
            c_values = "zero"
        cv = _draw(rng_c, (M, N), c_values)
        D[:, :N] = cv if out_dtype == F32 else to_bits16(cv, out_dtype)
        C = D
    else:
        D = _out_buffer(M, ldd, out_dtype)
        if c_values is not None:
            ldc = max(1, N) if ldc is None else ldc
            C = _out_buffer(M, ldc, out_dtype)
            cv = _draw(rng_c, (M, N), c_values)
            C[:, :N] = cv if out_dtype == F32 else to_bits16(cv, out_dtype)
        else:
            ldc = max(1, N) if ldc is None else ldc
    return Problem(name, M, N, K, A, lda, layoutA, B, ldb, layoutB, C, ldc, D, ldd,
                   in_dtype, acc_dtype, out_dtype, satf, inplace)


def scale_rows(prob: Problem, frac: float, factor: float, seed: int) -> np.ndarray:
    """Multiply round(frac*M) seeded rows of A by `factor` (a power of two, so
    the fp16 values stay exact).  Returns the chosen row indices."""
    rng = np.random.default_rng(seed)
    nrows = int(round(frac * prob.M))
    rows = np.sort(rng.choice(prob.M, size=nrows, replace=False))
    if prob.layoutA != ROW_MAJOR:
        raise ValueError("row scaling implemented for row-major A")
    vals = from_bits16(prob.A[rows, :prob.K], prob.in_dtype) * np.float32(factor)
    prob.A[rows, :prob.K] = to_bits16(vals, prob.in_dtype)
    return rows


def pattern_int(r, k):
    """X(r, k) = (131r + 71k + rk mod 97) mod 5 - 2 for broadcastable 64-bit
    integer arrays r, k (numpy or torch, on any device): integer values in
    [-2, 2], exact in every input type, with no short period along r or k,
    that need no storage to reproduce -- for operands too large to draw and
    keep on the host (any rows of them can be rebuilt for the oracle)."""
    return (131 * r + 71 * k + (r * k) % 97) % 5 - 2


def sample_indices(M: int, N: int, count: int, seed: int):
    """Seeded (row, col) pairs, without repetition when count <= M*N."""
    rng = np.random.default_rng(seed)
    total = M * N
    if count >= total:
        flat = np.arange(total, dtype=np.int64)
    else:
        flat = np.sort(rng.choice(total, size=count, replace=False)).astype(np.int64)
    return flat // N, flat % N


# ---------------------------------------------------------------------------
# The named workloads.  seed = 20260 + 10*index (+0 A, +1 B, +2 C; +3 scaled
# rows; +4 output sample).

def _seed(index: int) -> int:
    return 20260 + 10 * index


def w_256(values="uniform") -> Problem:
    """256^3, fp16 row-major in, C = 0, fp32 out."""
    return make_problem(256, 256, 256, values=values, seed=_seed(1),
                        name="256^3 fp16->fp32 (%s)" % values)


def w_4096_f16(values="uniform") -> Problem:
    """4096^3, fp16 row-major A and B, fp32 accumulate and output, C = 0."""
    return make_problem(4096, 4096, 4096, values=values, seed=_seed(2),
                        name="4096^3 fp16->fp32 (%s)" % values)


def w_4096_bf16_inplace(values="normal") -> Problem:
    """4096^3, bf16 row-major A, bf16 col-major B, C fp32 N(0,1) updated in place."""
    return make_problem(4096, 4096, 4096, layoutA=ROW_MAJOR, layoutB=COL_MAJOR,
                        in_dtype=BF16, values=values, c_values="normal", inplace=True,
                        seed=_seed(3), name="4096^3 bf16 colB inplace (%s)" % values)


def w_hgemm(satf: int, values="uniform", factor=None) -> Problem:
    """HGEMM 3999 x 4001 x 4104, fp16 accumulate/out, padded ld, 1% of A's rows
    scaled (x2048 uniform, x256 integer) to force overflow.  C = 0."""
    if factor is None:
        factor = 2048.0 if values == "uniform" else 256.0
    p = make_problem(3999, 4001, 4104, in_dtype=F16, acc_dtype=F16, out_dtype=F16,
                     satf=satf, values=values, c_values=None, lda=4104, ldb=4008,
                     ldc=4008, ldd=4008, seed=_seed(4),
                     name="HGEMM 3999x4001x4104 satf=%d (%s)" % (satf, values))
    # C: the workload names ldc but no C values; C = 0 (explicit zero buffer)
    p.C = np.zeros((p.M, p.ldc), dtype=np.uint16)
    p.extra["scaled_rows"] = scale_rows(p, 0.01, factor, _seed(4) + 3)
    return p


def w_wide(values="uniform") -> Problem:
    """16384 x 16384 x 1024, fp16 row-major in, fp32 out (sampled check)."""
    return make_problem(16384, 16384, 1024, values=values, seed=_seed(5),
                        name="16384x16384x1024 fp16->fp32 (%s)" % values)


def w_skinny(values="uniform") -> Problem:
    """16 x 16384 x 16384, fp16 row-major in, fp32 out (sampled check)."""
    return make_problem(16, 16384, 16384, values=values, seed=_seed(6),
                        name="16x16384x16384 fp16->fp32 (%s)" % values)


# ------------------------------------------------ extended-epilogue problems

@dataclasses.dataclass
class EpilogueProblem:
    """Inputs of one gemm_run_ex call: D = act(alpha * A x B + beta * C + bias)
    with C and D each row- or column-major.

    C and D buffers have shape (outer, ld): outer = M (row-major) or N
    (column-major).  ``bias`` is N float32 values or None."""
    name: str
    M: int
    N: int
    K: int
    A: np.ndarray
    lda: int
    layoutA: int
    B: np.ndarray
    ldb: int
    layoutB: int
    C: Optional[np.ndarray]
    ldc: int
    layoutC: int
    D: np.ndarray
    ldd: int
    layoutD: int
    in_dtype: int
    acc_dtype: int
    out_dtype: int
    satf: int
    alpha: float
    beta: float
    bias: Optional[np.ndarray]
    act: int
    inplace: bool = False

    @property
    def flops(self) -> int:
        return 2 * self.M * self.N * self.K


def make_epilogue_problem(M: int, N: int, K: int, *, layoutA=ROW_MAJOR, layoutB=ROW_MAJOR,
                          layoutC=ROW_MAJOR, layoutD=ROW_MAJOR, in_dtype=F16, acc_dtype=F32,
                          out_dtype=F32, satf=0, values="uniform",
                          c_values: Optional[str] = "normal", bias_values: Optional[str] = "normal",
                          alpha=1.0, beta=1.0, act=0, inplace=False, ldc=None, ldd=None,
                          seed=4321, name="epilogue", align=1) -> EpilogueProblem:
    """Seeded inputs for the extended epilogue (same value recipes as
    make_problem; the bias is drawn in fp32).  c_values=None: C = NULL.
    lda / ldb: the line length rounded up to a multiple of ``align``."""
    rng_a = np.random.default_rng(seed)
    rng_b = np.random.default_rng(seed + 1)
    rng_c = np.random.default_rng(seed + 2)
    rng_bias = np.random.default_rng(seed + 5)
    a_outer, a_inner = (M, K) if layoutA == ROW_MAJOR else (K, M)
    b_outer, b_inner = (K, N) if layoutB == ROW_MAJOR else (N, K)
    lda, ldb = _round_up(max(1, a_inner), align), _round_up(max(1, b_inner), align)
    A = _operand(rng_a, a_outer, a_inner, lda, in_dtype, values)
    B = _operand(rng_b, b_outer, b_inner, ldb, in_dtype, values)
    d_outer, d_inner = (M, N) if layoutD == ROW_MAJOR else (N, M)
    ldd = max(1, d_inner) + 3 if ldd is None else ldd
    D = _out_buffer(d_outer, ldd, out_dtype)
    C = None
    if inplace:
        layoutC, ldc = layoutD, ldd
        cv = _draw(rng_c, (d_outer, d_inner), c_values or "zero")
        D[:, :d_inner] = cv if out_dtype == F32 else to_bits16(cv, out_dtype)
        C = D
    elif c_values is not None:
        c_outer, c_inner = (M, N) if layoutC == ROW_MAJOR else (N, M)
        ldc = max(1, c_inner) + 1 if ldc is None else ldc
        C = _out_buffer(c_outer, ldc, out_dtype)
        cv = _draw(rng_c, (c_outer, c_inner), c_values)
        C[:, :c_inner] = cv if out_dtype == F32 else to_bits16(cv, out_dtype)
    else:
        ldc = max(1, N if layoutC == ROW_MAJOR else M) if ldc is None else ldc
    bias = None if bias_values is None else _draw(rng_bias, (N,), bias_values)
    return EpilogueProblem(name, M, N, K, A, lda, layoutA, B, ldb, layoutB, C, ldc, layoutC,
                           D, ldd, layoutD, in_dtype, acc_dtype, out_dtype, satf,
                           float(alpha), float(beta), bias, int(act), inplace)


# ------------------------------------------------ int8 x int8 -> int32 problems

I8, I32 = 3, 4
PAD_I8 = np.int8(-128)          # A/B padding: changes any sum that reads it
SENTINEL_I32 = np.int32(0x5A5A5A5A)


def _int8_operand(rng, rows: int, cols: int, ld: int, values: str) -> np.ndarray:
    buf = np.full((rows, ld), PAD_I8, dtype=np.int8)
    if rows and cols:
        lo, hi = (-128, 128) if values == "full" else (-3, 4)
        buf[:, :cols] = rng.integers(lo, hi, size=(rows, cols)).astype(np.int8)
    return buf


def make_int8_problem(M: int, N: int, K: int, *, layoutA=ROW_MAJOR, layoutB=COL_MAJOR,
                      values="full", c_values: Optional[str] = None, inplace=False, satf=0,
                      lda=None, ldb=None, ldc=None, ldd=None, seed=7777,
                      name="int8") -> Problem:
    """Seeded int8 A, B (``full``: uniform over [-128, 127]; ``small``: [-3, 3])
    and int32 C (``int``: [-1000, 1000]; ``big``: the whole int32 range), all
    row-major C/D.  A/B padding holds -128, D a sentinel."""
    rng_a = np.random.default_rng(seed)
    rng_b = np.random.default_rng(seed + 1)
    rng_c = np.random.default_rng(seed + 2)
    a_outer, a_inner = (M, K) if layoutA == ROW_MAJOR else (K, M)
    b_outer, b_inner = (K, N) if layoutB == ROW_MAJOR else (N, K)
    lda = max(1, a_inner) if lda is None else lda
    ldb = max(1, b_inner) if ldb is None else ldb
    ldd = max(1, N) if ldd is None else ldd
    A = _int8_operand(rng_a, a_outer, a_inner, lda, values)
    B = _int8_operand(rng_b, b_outer, b_inner, ldb, values)
    D = np.full((M, ldd), SENTINEL_I32, dtype=np.int32)

    def draw_c(shape):
        if c_values == "big":
            return rng_c.integers(-2 ** 31, 2 ** 31, size=shape, dtype=np.int64).astype(np.int32)
        return rng_c.integers(-1000, 1001, size=shape).astype(np.int32)

    C = None
    if inplace:
        ldc = ldd
        D[:, :N] = draw_c((M, N))
        C = D
    elif c_values is not None:
        ldc = max(1, N) if ldc is None else ldc
        C = np.full((M, ldc), SENTINEL_I32, dtype=np.int32)
        C[:, :N] = draw_c((M, N))
    else:
        ldc = max(1, N) if ldc is None else ldc
    return Problem(name, M, N, K, A, lda, layoutA, B, ldb, layoutB, C, ldc, D, ldd,
                   I8, I32, I32, satf, inplace)
