"""gemm_run_noalloc (no device allocation: split-K partial sums in the
library's fixed scratch) against gemm_run through the C ABI: two calls in a
row, the second with a smaller problem, each bit-identical to gemm_run (the
same kernels and split) and within the oracle's bounds; and captured into a
HIP graph and replayed.  Runs alone in a fresh process and after the other
GPU tests."""
import numpy as np
import pytest
import torch

import dense_mixed_precision_tiled_amd as lg
from dense_mixed_precision_tiled_amd import workloads as W
from gpu_util import DeviceProblem, compare, log, oracle_whole, region

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    lg.library()
    yield


def _run(dp, fn):
    p = dp.prob
    dp.reset_D()
    st = fn(p.M, p.N, p.K, dp.A.data_ptr(), p.lda, p.layoutA, dp.B.data_ptr(), p.ldb, p.layoutB,
            None if dp.C is None else dp.C.data_ptr(), p.ldc, dp.D.data_ptr(), p.ldd,
            p.in_dtype, p.acc_dtype, p.out_dtype, p.satf,
            torch.cuda.current_stream().cuda_stream)
    assert st == 0, lg.gemm_status_string(st)
    return dp.result().copy()


@pytest.mark.parametrize("values,exact", [("int", True), ("uniform", False)])
def test_noalloc_matches_gemm_run_on_two_calls_second_smaller(values, exact):
    # split-K (M <= 16) problems: the first needs the larger share of the
    # scratch, the second a smaller one that reuses it; then a problem with no
    # split at all
    probs = [W.make_problem(16, 8192, 16384, values=values, c_values="normal" if not exact
                            else "int", seed=7100, name="16x8192x16384 +C"),
             W.make_problem(9, 3000, 5000, values=values, ldd=3003, seed=7101,
                            name="9x3000x5000"),
             W.make_problem(300, 257, 129, values=values, ldd=260, seed=7102,
                            name="300x257x129")]
    for prob in probs:
        log("case: gemm_run_noalloc %s %s" % (prob.name, values))
        dp = DeviceProblem(prob)
        want = _run(dp, lg.gemm_run)
        got = _run(dp, lg.gemm_run_noalloc)
        assert np.array_equal(got.view(np.uint8), want.view(np.uint8)), prob.name
        compare(prob, region(prob, got), region(prob, oracle_whole(prob)), exact,
                label="noalloc " + prob.name)


def _args(dp):
    p = dp.prob
    return (p.M, p.N, p.K, dp.A.data_ptr(), p.lda, p.layoutA, dp.B.data_ptr(), p.ldb, p.layoutB,
            None if dp.C is None else dp.C.data_ptr(), p.ldc, dp.D.data_ptr(), p.ldd,
            p.in_dtype, p.acc_dtype, p.out_dtype, p.satf)


def _eager(dp, fn):
    dp.reset_D()
    st = fn(*_args(dp), torch.cuda.current_stream().cuda_stream)
    assert st == 0, lg.gemm_status_string(st)
    return dp.result().copy()


@pytest.mark.parametrize("shape", [(16, 4096, 8192), (520, 530, 384)])
def test_noalloc_replayed_from_a_graph(shape):
    """The callers gemm_run_noalloc is for include code under graph capture:
    captured once (the split-K shape captures the partial-sum kernel and the
    reduction over the library's scratch), replayed three times with eager
    calls of both entry points on other data between the replays (the same
    scratch), every replay equals the eager result bit for bit."""
    M, N, K = shape
    dp = DeviceProblem(W.make_problem(M, N, K, values="int", c_values="int", seed=7200 + M))
    dq = DeviceProblem(W.make_problem(M, N, K, values="int", c_values="int", seed=7300 + M))
    want = _eager(dp, lg.gemm_run_noalloc)
    other = _eager(dq, lg.gemm_run_noalloc)
    log("case: graph capture of gemm_run_noalloc %dx%dx%d" % shape)
    dp.reset_D()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        st = lg.gemm_run_noalloc(*_args(dp), torch.cuda.current_stream().cuda_stream)
    assert st == 0, lg.gemm_status_string(st)
    for rep in range(3):
        eager = _eager(dq, lg.gemm_run_noalloc if rep % 2 == 0 else lg.gemm_run)
        assert np.array_equal(eager.view(np.uint8), other.view(np.uint8)), rep
        dp.reset_D()
        torch.cuda.synchronize()
        g.replay()
        got = dp.result().copy()
        assert np.array_equal(got.view(np.uint8), want.view(np.uint8)), "replay %d" % rep
