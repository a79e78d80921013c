"""Helpers for the GPU parity tests: move a seeded Problem to the device, run
it through the C ABI, and compare with the CPU oracle to the stated bar.

Tolerances (written here, derived in the design notes):
  fp32 out : per element |err| <= 1e-4*sqrt(K), relative Frobenius <= 1e-5
  fp16 out : per element |err| <= 2^-10*|ref| + 2e-3*sqrt(K); where the exact
             value lies within that bound of the fp16 overflow threshold 65520,
             +-65504 and +-Inf of the same sign are both accepted
  bf16 out : per element |err| <= 2^-7*|ref| + 1e-4*sqrt(K) (one bf16 ulp from
             rounding an fp32 sum instead of the exact one, plus the fp32 bound)
  integer-valued inputs: bit-exact (IEEE equality; NaN positions equal)
  fp8 inputs: the bounds above plus K * 2^-13 * max|a| * max|b|
             (fp8_block_bound), relative Frobenius <= 2^-12
"""
from __future__ import annotations

import math
import sys

import numpy as np
import torch

import dense_mixed_precision_tiled_amd as lg
import oracle
from dense_mixed_precision_tiled_amd.workloads import (BF16, F16, F32, FP8_E4M3, FP8_E5M2, I8,
                                                       SENTINEL_16, SENTINEL_F32, from_bits16)


def log(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def _dev(x: np.ndarray) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(x).view(np.int16 if x.dtype == np.uint16
                                                      else x.dtype))
    return t.to("cuda")


def _host(t: torch.Tensor, like: np.ndarray) -> np.ndarray:
    return t.cpu().numpy().view(like.dtype).reshape(like.shape)


class DeviceProblem:
    """Device copies of a Problem's buffers (C aliases D when in place)."""

    def __init__(self, prob):
        self.prob = prob
        self.A = _dev(prob.A)
        self.B = _dev(prob.B)
        self.D = _dev(prob.D)
        if prob.inplace:
            self.C = self.D
        elif prob.C is not None:
            self.C = _dev(prob.C)
        else:
            self.C = None

    def reset_D(self):
        self.D.copy_(_dev(self.prob.D))

    def run(self, config=None, stream=None, satf=None):
        p = self.prob
        s = (stream or torch.cuda.current_stream()).cuda_stream
        args = (p.M, p.N, p.K, self.A.data_ptr(), p.lda, p.layoutA, self.B.data_ptr(), p.ldb,
                p.layoutB, None if self.C is None else self.C.data_ptr(), p.ldc,
                self.D.data_ptr(), p.ldd, p.in_dtype, p.acc_dtype, p.out_dtype,
                p.satf if satf is None else satf, s)
        st = lg.gemm_run(*args) if config is None else lg.gemm_run_config(config, *args)
        if st != 0:
            raise lg.GemmError(st)
        return st

    def result(self) -> np.ndarray:
        torch.cuda.synchronize()
        return _host(self.D, self.prob.D)

    def gather(self, rows, cols) -> np.ndarray:
        """D(rows[s], cols[s]) copied back, gathered on the device."""
        torch.cuda.synchronize()
        p = self.prob
        flat = torch.from_numpy(np.asarray(rows, np.int64) * p.ldd + np.asarray(cols, np.int64))
        vals = self.D.reshape(-1)[flat.to("cuda")].cpu().numpy()
        return vals.view(p.D.dtype)


def oracle_full(prob) -> np.ndarray:
    """The oracle's D buffer (full M x N region; padding keeps the sentinel)."""
    D = prob.D.copy()
    C = D if prob.inplace else prob.C
    oracle.gemm(prob.M, prob.N, prob.K, prob.A.ravel(), prob.lda, prob.layoutA,
                prob.B.ravel(), prob.ldb, prob.layoutB,
                None if C is None else C.ravel(), prob.ldc, D.ravel(), prob.ldd,
                prob.in_dtype, prob.acc_dtype, prob.out_dtype, prob.satf)
    return D


def oracle_whole(prob, sums=None) -> np.ndarray:
    """The whole D buffer by the oracle's product form (fp64 library matmul of
    the exactly decoded operands, then the C oracle's epilogue, rounding and
    satf) -- the oracle for full outputs of the large workloads.  Works for
    Problem (plain), EpilogueProblem (extended epilogue) and int8 problems;
    padding keeps its sentinel.  ``sums``: precomputed product sums (reused
    between calls that differ only in satf)."""
    D = prob.D.copy()
    C = D if prob.inplace else prob.C
    Cf = None if C is None else C.ravel()
    if prob.in_dtype == I8:
        oracle.gemm_i8_product(prob.M, prob.N, prob.K, prob.A.ravel(), prob.lda, prob.layoutA,
                               prob.B.ravel(), prob.ldb, prob.layoutB, Cf, prob.ldc,
                               getattr(prob, "layoutC", 0), D.ravel(), prob.ldd,
                               getattr(prob, "layoutD", 0), prob.satf)
        return D
    ex = {}
    if hasattr(prob, "act"):
        ex = dict(layoutC=prob.layoutC, layoutD=prob.layoutD, alpha=prob.alpha, beta=prob.beta,
                  bias=prob.bias, act=prob.act)
    oracle.gemm_product(prob.M, prob.N, prob.K, prob.A.ravel(), prob.lda, prob.layoutA,
                        prob.B.ravel(), prob.ldb, prob.layoutB, Cf, prob.ldc, D.ravel(), prob.ldd,
                        prob.in_dtype, prob.acc_dtype, prob.out_dtype, prob.satf, sums=sums, **ex)
    return D


def product_sums(prob) -> np.ndarray:
    """sum_k A(i,k) B(k,j) in fp64 (M x N) by the oracle's product form."""
    return oracle.product_sums(prob.M, prob.N, prob.K, prob.A.ravel(), prob.lda, prob.layoutA,
                               prob.B.ravel(), prob.ldb, prob.layoutB, prob.in_dtype)


def oracle_samples(prob, rows, cols) -> np.ndarray:
    C = prob.D if prob.inplace else prob.C  # prob.D still holds the original C
    return oracle.gemm_sampled(prob.M, prob.N, prob.K, prob.A.ravel(), prob.lda, prob.layoutA,
                               prob.B.ravel(), prob.ldb, prob.layoutB,
                               None if C is None else C.ravel(), prob.ldc, rows, cols,
                               prob.in_dtype, prob.acc_dtype, prob.out_dtype, prob.satf)


def fp8_block_bound(prob) -> float:
    """Extra tolerance for fp8 inputs: the fp8 MFMA adds its products in
    groups of 8 aligned to the largest of each group, and what lies below
    2^-13 of that largest product is lost (pinned on the instruction by
    test_fp8_gpu.test_fp8_group_truncation).  So each product is off by less
    than 2^-13 * max|a| * max|b|: K products."""
    dec = oracle.decode_fp8_e4m3 if prob.in_dtype == FP8_E4M3 else oracle.decode_fp8_e5m2
    table = np.array([dec(b) for b in range(256)])
    table[np.isnan(table)] = 0.0
    ka = prob.K if prob.layoutA == 0 else prob.M
    kb = prob.N if prob.layoutB == 0 else prob.K
    amax = np.abs(table[prob.A[:, :ka]]).max() if prob.A.size else 0.0
    bmax = np.abs(table[prob.B[:, :kb]]).max() if prob.B.size else 0.0
    return max(prob.K, 0) * 2.0 ** -13 * amax * bmax


def values(x: np.ndarray, out_dtype: int) -> np.ndarray:
    if out_dtype == F32:
        return x.astype(np.float64)
    return from_bits16(x, out_dtype).astype(np.float64)


def compare(prob, got, ref, exact: bool, rows=None, cols=None, label=""):
    """got/ref: out_dtype element arrays of equal shape (region or samples).
    Raises AssertionError with the first offending elements."""
    K = prob.K
    g = values(np.asarray(got), prob.out_dtype).ravel()
    r = values(np.asarray(ref), prob.out_dtype).ravel()
    nan_g, nan_r = np.isnan(g), np.isnan(r)
    assert np.array_equal(nan_g, nan_r), "%s: NaN positions differ (%d vs %d)" % (
        label, nan_g.sum(), nan_r.sum())
    ok = ~nan_r
    g, r = g[ok], r[ok]
    if exact:
        bad = np.nonzero(g != r)[0]
        assert bad.size == 0, "%s: %d of %d not bit-exact, e.g. got %s ref %s" % (
            label, bad.size, g.size, g[bad[:5]], r[bad[:5]])
        return
    root = math.sqrt(max(K, 0))
    if prob.out_dtype == F32:
        bound = np.full_like(r, 1e-4 * root)
    elif prob.out_dtype == F16:
        bound = 2.0 ** -10 * np.abs(r) + 2e-3 * root
    else:
        bound = 2.0 ** -7 * np.abs(r) + 1e-4 * root
    if prob.in_dtype in (FP8_E4M3, FP8_E5M2):
        bound = bound + fp8_block_bound(prob)
    inf_g, inf_r = np.isinf(g), np.isinf(r)
    fin = ~inf_g & ~inf_r
    err = np.abs(g[fin] - r[fin])
    badf = np.nonzero(err > bound[fin])[0]
    # overflow classification near the fp16 threshold
    special = np.nonzero(inf_g | inf_r)[0]
    bad_special = []
    if special.size:
        idx = np.nonzero(ok)[0][special]
        for s_i, flat in zip(special, idx):
            gv, rv = g[s_i], r[s_i]
            if gv == rv:
                continue
            if prob.out_dtype == F16 and np.sign(gv) == np.sign(rv) and \
                    abs(gv) >= 65504 and abs(rv) >= 65504:
                i, j = (rows[flat], cols[flat]) if rows is not None else divmod(flat, prob.N)
                C = prob.D if prob.inplace else prob.C
                s = oracle.element_fp64(prob.K, prob.A.ravel(), prob.lda, prob.layoutA,
                                        prob.B.ravel(), prob.ldb, prob.layoutB,
                                        None if C is None else C.ravel(), prob.ldc,
                                        prob.in_dtype, prob.out_dtype, int(i), int(j))
                band = 2.0 ** -10 * 65520 + 2e-3 * root
                if abs(abs(s) - 65520.0) <= band:
                    continue
            bad_special.append((gv, rv))
    assert badf.size == 0, "%s: %d of %d beyond tolerance, e.g. got %s ref %s bound %s" % (
        label, badf.size, err.size, g[fin][badf[:5]], r[fin][badf[:5]], bound[fin][badf[:5]])
    assert not bad_special, "%s: Inf mismatch %s" % (label, bad_special[:5])
    if prob.out_dtype == F32 and fin.any():
        # fp8 inputs: the MFMA drops what lies below 2^-13 of the largest
        # product of each group of 8; on the tests' random data that
        # averages far below 2^-12 of the result's norm
        rel_bar = 2.0 ** -12 if prob.in_dtype in (FP8_E4M3, FP8_E5M2) else 1e-5
        nr = np.linalg.norm(r[fin])
        if nr > 0:
            rel = np.linalg.norm(g[fin] - r[fin]) / nr
            assert rel <= rel_bar, "%s: relative Frobenius error %.3g > %.3g" % (label, rel,
                                                                                 rel_bar)


def region(prob, D: np.ndarray) -> np.ndarray:
    return D[:prob.M, :prob.N]


def check_padding(prob, D: np.ndarray, label=""):
    """Columns N..ldd-1 of D still hold the sentinel (in place: C's padding)."""
    if prob.ldd > prob.N:
        pad = D[:prob.M, prob.N:]
        want = prob.D[:prob.M, prob.N:]
        assert np.array_equal(pad.view(np.uint8), want.view(np.uint8)), \
            "%s: D padding was written" % label
