"""GPU parity of the extended epilogue, D = act(alpha * A x B + beta * C + bias),
with row- or column-major C and D, through the C ABI (gemm_run_ex /
gemm_run_ex_config) against the oracle's gemm_ex.

Tolerance for non-integer data (derived in the design notes): with S the
exact product sum, x = alpha*S + beta*C + bias the pre-activation value and
L the activation's Lipschitz constant (1 for none/ReLU, 1.13 for GELU),
    |err| <= L * (|alpha| * T + 2^-21 * (|alpha*S| + |beta*C| + |bias|))
             + 2^-20 * |ref| + R * |ref|
where T is the accumulation bound of the plain path (1e-4*sqrt(K) for fp32
and bf16 outputs, 2e-3*sqrt(K) for fp16) and R the output rounding (0 for
fp32, 2^-10 fp16, 2^-7 bf16).  The 2^-21 term covers the fp32 scaling, adds
and GELU evaluation (erff) between the accumulator and the final rounding.
Integer data with dyadic alpha/beta and integer bias is bit-exact.
"""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import dense_mixed_precision_tiled_amd as lg
import oracle
from dense_mixed_precision_tiled_amd import workloads as W
from dense_mixed_precision_tiled_amd.workloads import BF16, COL_MAJOR, F16, F32, ROW_MAJOR
from gpu_util import log, oracle_whole, product_sums, values

pytestmark = pytest.mark.gpu

NONE, RELU, GELU = lg.GEMM_ACT_NONE, lg.GEMM_ACT_RELU, lg.GEMM_ACT_GELU
# tile-table entry -> block tile edge (None: skinny split-K), as in test_gemm_gpu
ENTRY_TILE = {0: 256, 1: 128, 2: 64, 3: None, 4: 256, 13: 256, 14: 32, 15: 256}
VEC_ONLY = {13, 15}   # LDS-DMA entries: 16-byte aligned operand lines only


def _align(cid):
    return 8 if cid in VEC_ONLY else 1


def _entry_shape(cid):
    bm = ENTRY_TILE[cid]
    return (13, 3 * 128 - 5, 1100) if bm is None else (2 * bm + 17, 3 * bm - 5, 200)


def _dev(x):
    if x is None:
        return None
    return torch.from_numpy(np.ascontiguousarray(x).view(
        np.int16 if x.dtype == np.uint16 else x.dtype)).to("cuda")


class Dev:
    def __init__(self, ep, bias_offset=0):
        self.ep = ep
        self.A, self.B, self.D = _dev(ep.A), _dev(ep.B), _dev(ep.D)
        self.C = self.D if ep.inplace else _dev(ep.C)
        self.bias = None
        if ep.bias is not None:
            # bias_offset > 0 places the bias at a non-16-byte-aligned address
            self.bias_buf = torch.zeros(ep.N + 4, dtype=torch.float32, device="cuda")
            self.bias_buf[bias_offset:bias_offset + ep.N] = torch.from_numpy(ep.bias).cuda()
            self.bias = self.bias_buf[bias_offset:]

    def epi(self):
        ep = self.ep
        return lg.GemmEpilogue(ep.alpha, ep.beta, 0 if self.bias is None else self.bias.data_ptr(),
                               ep.act, ep.layoutC, ep.layoutD)

    def run(self, config=None, epi="ex"):
        ep = self.ep
        args = (ep.M, ep.N, ep.K, self.A.data_ptr(), ep.lda, ep.layoutA, self.B.data_ptr(),
                ep.ldb, ep.layoutB, None if self.C is None else self.C.data_ptr(), ep.ldc,
                self.D.data_ptr(), ep.ldd, ep.in_dtype, ep.acc_dtype, ep.out_dtype, ep.satf)
        s = torch.cuda.current_stream().cuda_stream
        e = self.epi() if epi == "ex" else None
        st = (lg.gemm_run_ex(*args, e, s) if config is None
              else lg.gemm_run_ex_config(config, *args, e, s))
        if st != 0:
            raise lg.GemmError(st, "gemm_run_ex")

    def result(self):
        torch.cuda.synchronize()
        return self.D.cpu().numpy().view(self.ep.D.dtype).reshape(self.ep.D.shape)


def oracle_ex(ep, alpha=None, beta=None, bias="same", act=None, out_dtype=None, layoutD=None):
    """The oracle's D buffer for ep (overrides compute auxiliary quantities)."""
    od = ep.out_dtype if out_dtype is None else out_dtype
    lD = ep.layoutD if layoutD is None else layoutD
    if out_dtype is None and layoutD is None:
        D = ep.D.copy()
        ldd = ep.ldd
    else:
        D = np.zeros((ep.M, ep.N) if lD == ROW_MAJOR else (ep.N, ep.M),
                     dtype=np.float32 if od == F32 else np.uint16)
        ldd = D.shape[1]
    C = D if (ep.inplace and out_dtype is None and layoutD is None) else \
        (ep.D.copy() if ep.inplace else ep.C)
    if (ep.beta if beta is None else beta) == 0:
        C = None  # beta = 0 reads no C (and C's dtype need not match an overridden out_dtype)
    oracle.gemm_ex(ep.M, ep.N, ep.K, ep.A.ravel(), ep.lda, ep.layoutA, ep.B.ravel(), ep.ldb,
                   ep.layoutB, None if C is None else C.ravel(), ep.ldc, ep.layoutC,
                   D.ravel(), ldd, lD, ep.in_dtype, ep.acc_dtype if od == ep.out_dtype else F32,
                   od, ep.satf, ep.alpha if alpha is None else alpha,
                   ep.beta if beta is None else beta, ep.bias if bias == "same" else bias,
                   ep.act if act is None else act)
    return D


def region(ep, D, layoutD=None):
    """The M x N matrix of a D buffer (row-major view)."""
    lD = ep.layoutD if layoutD is None else layoutD
    return D[:ep.M, :ep.N] if lD == ROW_MAJOR else D[:ep.N, :ep.M].T


def c_values(ep):
    """|C(i,j)| as an M x N float64 array (0 where C is absent)."""
    if ep.C is None:
        return np.zeros((ep.M, ep.N))
    Cb = ep.C if not ep.inplace else ep.D
    m = region(ep, Cb, ep.layoutC)
    return np.abs(values(np.asarray(m), ep.out_dtype).reshape(ep.M, ep.N))


def compare_ex(ep, got, ref, exact, label):
    g = values(np.ascontiguousarray(region(ep, got)), ep.out_dtype).reshape(ep.M, ep.N)
    r = values(np.ascontiguousarray(region(ep, ref)), ep.out_dtype).reshape(ep.M, ep.N)
    assert np.array_equal(np.isnan(g), np.isnan(r)), "%s: NaN positions differ" % label
    ok = ~np.isnan(r)
    if exact:
        bad = np.argwhere(ok & (g != r))
        assert bad.size == 0, "%s: %d not bit-exact, e.g. %s got %s ref %s" % (
            label, len(bad), bad[:3].tolist(), g[tuple(bad[:3].T)], r[tuple(bad[:3].T)])
    else:
        S = oracle_ex(ep, alpha=1.0, beta=0.0, bias=None, act=NONE, out_dtype=F32,
                      layoutD=ROW_MAJOR).astype(np.float64)
        bias = np.zeros(ep.N) if ep.bias is None else np.abs(ep.bias.astype(np.float64))
        root = math.sqrt(max(ep.K, 0))
        T = (2e-3 if ep.out_dtype == F16 else 1e-4) * root
        R = {F32: 0.0, F16: 2.0 ** -10, BF16: 2.0 ** -7}[ep.out_dtype]
        L = 1.13 if ep.act == GELU else 1.0
        beta_c = abs(ep.beta) * c_values(ep) if ep.beta != 0 else 0.0
        bound = (L * (abs(ep.alpha) * T + 2.0 ** -21 * (abs(ep.alpha) * np.abs(S) + beta_c +
                                                        bias[None, :]))
                 + (2.0 ** -20 + R) * np.abs(r))
        fin = ok & np.isfinite(r) & np.isfinite(g)
        assert np.array_equal(np.isinf(g) & ok, np.isinf(r) & ok), "%s: Inf positions" % label
        assert np.array_equal(g[np.isinf(r)], r[np.isinf(r)]), "%s: Inf signs" % label
        err = np.abs(g - r)
        bad = np.argwhere(fin & (err > bound))
        assert bad.size == 0, "%s: %d beyond tolerance, e.g. %s got %s ref %s bound %s" % (
            label, len(bad), bad[:3].tolist(), g[tuple(bad[:3].T)], r[tuple(bad[:3].T)],
            bound[tuple(bad[:3].T)])
    # nothing outside the M x N region of D was written
    inner = ep.N if ep.layoutD == ROW_MAJOR else ep.M
    outer = ep.M if ep.layoutD == ROW_MAJOR else ep.N
    pad_g, pad_r = got[:outer, inner:], ep.D[:outer, inner:]
    assert np.array_equal(pad_g.view(np.uint8), pad_r.view(np.uint8)), "%s: padding" % label
    assert np.array_equal(got[outer:].view(np.uint8), ep.D[outer:].view(np.uint8))


def _check(ep, exact, config=None, label="", bias_offset=0):
    log("case: %s config=%s" % (label, config))
    d = Dev(ep, bias_offset)
    d.run(config)
    compare_ex(ep, d.result(), oracle_ex(ep), exact, label)


LAYOUTS_CD = [(ROW_MAJOR, ROW_MAJOR), (COL_MAJOR, COL_MAJOR), (ROW_MAJOR, COL_MAJOR),
              (COL_MAJOR, ROW_MAJOR)]


@pytest.mark.parametrize("cid", sorted(ENTRY_TILE))
@pytest.mark.parametrize("lc,ld", LAYOUTS_CD)
def test_every_entry_gelu_bias_scale(cid, lc, ld):
    M, N, K = _entry_shape(cid)
    ep = W.make_epilogue_problem(M, N, K, layoutA=ROW_MAJOR, layoutB=ROW_MAJOR, layoutC=lc,
                                 layoutD=ld, values="uniform", c_values="normal",
                                 bias_values="normal", alpha=0.75, beta=-0.5, act=GELU,
                                 seed=5000 + cid, align=_align(cid))
    _check(ep, False, cid, "cfg%d GELU C%d D%d" % (cid, lc, ld))


@pytest.mark.parametrize("cid", sorted(ENTRY_TILE))
@pytest.mark.parametrize("out_dt,acc_dt,in_dt", [(F32, F32, F16), (F16, F16, F16),
                                                 (BF16, F32, BF16)])
def test_every_entry_relu_integer_exact(cid, out_dt, acc_dt, in_dt):
    M, N, K = _entry_shape(cid)
    la, lb = (COL_MAJOR, ROW_MAJOR) if cid % 2 else (ROW_MAJOR, COL_MAJOR)
    ep = W.make_epilogue_problem(M, N, K, layoutA=la, layoutB=lb, layoutC=ROW_MAJOR,
                                 layoutD=COL_MAJOR if cid % 2 == 0 else ROW_MAJOR,
                                 in_dtype=in_dt, acc_dtype=acc_dt, out_dtype=out_dt,
                                 values="int", c_values="int", bias_values="int",
                                 alpha=2.0, beta=-1.0, act=RELU, satf=1, seed=5100 + cid,
                                 align=_align(cid))
    _check(ep, True, cid, "cfg%d ReLU int out=%d" % (cid, out_dt))


@pytest.mark.parametrize("cid", sorted(ENTRY_TILE))
@pytest.mark.parametrize("out_dt,acc_dt", [(F32, F32), (F16, F16), (BF16, F32)])
@pytest.mark.parametrize("lcd", [ROW_MAJOR, COL_MAJOR])
def test_every_entry_vector_epilogue_with_c_and_bias(cid, out_dt, acc_dt, lcd):
    """alpha, beta * C, bias and an activation with row-major C and D whose
    leading dimensions are multiples of 4 (vector C/D/bias access): the staged
    pre-phase applies the linear part to the groups inside M x N, the groups
    crossing column N take the element path.  Integer data, bit-exact; then
    uniform data with GELU."""
    M, N, K = _entry_shape(cid)
    # column-major C and D run as the transposed problem, with the bias per row
    ld = (max(M, N) + 3) // 4 * 4 + 4
    ep = W.make_epilogue_problem(M, N, K, layoutA=ROW_MAJOR, layoutB=ROW_MAJOR, layoutC=lcd,
                                 layoutD=lcd, out_dtype=out_dt, acc_dtype=acc_dt, values="int",
                                 c_values="int", bias_values="int", alpha=2.0, beta=-1.0,
                                 act=RELU, ldc=ld, ldd=ld, seed=5300 + cid, align=_align(cid))
    _check(ep, True, cid, "cfg%d vector epilogue int out=%d CD%d" % (cid, out_dt, lcd))
    ep = W.make_epilogue_problem(M, N, K, layoutA=ROW_MAJOR, layoutB=ROW_MAJOR, layoutC=lcd,
                                 layoutD=lcd, out_dtype=out_dt, acc_dtype=acc_dt,
                                 values="uniform", c_values="normal", bias_values="normal",
                                 alpha=0.75, beta=-0.5, act=GELU, ldc=ld, ldd=ld,
                                 seed=5350 + cid, align=_align(cid))
    _check(ep, False, cid, "cfg%d vector epilogue GELU out=%d CD%d" % (cid, out_dt, lcd))


@pytest.mark.parametrize("layout", [ROW_MAJOR, COL_MAJOR])
def test_in_place(layout):
    ep = W.make_epilogue_problem(300, 257, 129, layoutC=layout, layoutD=layout, inplace=True,
                                 values="int", c_values="int", bias_values="int",
                                 alpha=1.0, beta=1.0, act=RELU, seed=5200 + layout)
    _check(ep, True, None, "in place layout %d" % layout)


def test_beta_zero_does_not_read_c():
    ep = W.make_epilogue_problem(200, 300, 64, values="int", c_values="int", bias_values="int",
                                 alpha=-1.0, beta=0.0, act=NONE, seed=5300)
    nan = np.float32(np.nan)
    ep.C[:] = nan  # poisoned: must not reach D
    d = Dev(ep)
    d.run()
    got = d.result()
    assert np.isfinite(region(ep, got)).all()
    compare_ex(ep, got, oracle_ex(ep), True, "beta 0")


@pytest.mark.parametrize("act", [NONE, RELU, GELU])
def test_k_zero(act):
    ep = W.make_epilogue_problem(70, 90, 0, layoutC=COL_MAJOR, layoutD=ROW_MAJOR,
                                 values="uniform", c_values="normal", bias_values="normal",
                                 alpha=3.0, beta=0.5, act=act, seed=5400 + act)
    _check(ep, False, None, "K=0 act %d" % act)


def test_unaligned_bias_takes_the_element_path():
    ep = W.make_epilogue_problem(520, 530, 96, values="int", c_values=None, bias_values="int",
                                 alpha=0.5, beta=1.0, act=RELU, seed=5500)
    _check(ep, True, None, "bias offset 1 float", bias_offset=1)


@pytest.mark.parametrize("cid", [0, 1, 4, 13, 15])
def test_default_epilogue_is_gemm_run(cid):
    prob = W.make_problem(700, 650, 300, layoutA=ROW_MAJOR, layoutB=COL_MAJOR, values="uniform",
                          c_values="normal", ldd=656, seed=5600 + cid, align=_align(cid))
    A, B = _dev(prob.A), _dev(prob.B)
    C = _dev(prob.C)
    outs = []
    for mode in ("run", "ex_none", "ex_default"):
        D = _dev(prob.D)
        args = (prob.M, prob.N, prob.K, A.data_ptr(), prob.lda, prob.layoutA, B.data_ptr(),
                prob.ldb, prob.layoutB, C.data_ptr(), prob.ldc, D.data_ptr(), prob.ldd,
                prob.in_dtype, prob.acc_dtype, prob.out_dtype, prob.satf)
        s = torch.cuda.current_stream().cuda_stream
        if mode == "run":
            st = lg.gemm_run_config(cid, *args, s)
        else:
            st = lg.gemm_run_ex_config(cid, *args,
                                       None if mode == "ex_none" else lg.GemmEpilogue(), s)
        assert st == 0
        torch.cuda.synchronize()
        outs.append(D.cpu().numpy().view(np.uint32))
    assert np.array_equal(outs[0], outs[1]) and np.array_equal(outs[0], outs[2])


@pytest.mark.parametrize("layoutD", [ROW_MAJOR, COL_MAJOR])
def test_4096_bias_gelu_whole_output(layoutD):
    """The 4096^3 fp16 workload with bias + GELU (alpha = 1, no C), as the
    benchmark times it: every output against the oracle's product form,
    within the extended-epilogue bound (S = the exact product sums)."""
    n = 4096
    ep = W.make_epilogue_problem(n, n, n, layoutD=layoutD, values="uniform", c_values=None,
                                 bias_values="normal", act=GELU, ldd=n, seed=5700 + layoutD)
    log("case: 4096 bias+GELU layoutD=%d (whole output)" % layoutD)
    d = Dev(ep)
    d.run()
    got = region(ep, d.result()).astype(np.float64)
    S = product_sums(ep)
    ref = region(ep, oracle_whole(ep, sums=S)).astype(np.float64)
    bias = ep.bias[None, :].astype(np.float64)   # region() is the M x N view for either layout
    bound = 1.13 * (1e-4 * math.sqrt(n) + 2.0 ** -21 * (np.abs(S) + np.abs(bias))) \
        + 2.0 ** -20 * np.abs(ref)
    err = np.abs(got - ref)
    assert np.isfinite(got).all()
    assert (err <= bound).all(), (err.max(), int(np.count_nonzero(err > bound)))
    rel = np.linalg.norm(got - ref) / np.linalg.norm(ref)
    assert rel <= 1e-5, rel
