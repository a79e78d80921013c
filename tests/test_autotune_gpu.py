"""GPU tests of the runtime autotuner (gemm_autotune): it picks a table entry,
records it for the problem signature, leaves a correct D, and later
gemm_run / gemm_run_ex calls with that signature run the recorded entry."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import dense_mixed_precision_tiled_amd as lg
import oracle
from dense_mixed_precision_tiled_amd import workloads as W
from dense_mixed_precision_tiled_amd.workloads import COL_MAJOR, F16, F32, ROW_MAJOR
from gpu_util import DeviceProblem, compare, log, oracle_full, region

pytestmark = pytest.mark.gpu


def _args(dp):
    p = dp.prob
    return (p.M, p.N, p.K, dp.A.data_ptr(), p.lda, p.layoutA, dp.B.data_ptr(), p.ldb,
            p.layoutB, None if dp.C is None else dp.C.data_ptr(), p.ldc, dp.D.data_ptr(), p.ldd,
            p.in_dtype, p.acc_dtype, p.out_dtype, p.satf)


def _bits(dp):
    return dp.result().view(np.uint32 if dp.prob.out_dtype == F32 else np.uint16).copy()


@pytest.mark.parametrize("shape,la,lb", [((1000, 1100, 300), ROW_MAJOR, ROW_MAJOR),
                                         ((16, 3000, 2048), ROW_MAJOR, COL_MAJOR),
                                         ((2100, 700, 520), COL_MAJOR, ROW_MAJOR)])
def test_autotune_records_and_dispatches(shape, la, lb):
    M, N, K = shape
    lg.gemm_autotune_clear()
    prob = W.make_problem(M, N, K, layoutA=la, layoutB=lb, values="uniform", c_values="normal",
                          ldd=N + 4, seed=6000 + M)
    log("case: autotune %dx%dx%d A%d B%d" % (M, N, K, la, lb))
    dp = DeviceProblem(prob)
    s = torch.cuda.current_stream().cuda_stream
    st, cfg = lg.gemm_autotune(*_args(dp), None, 3, s)
    assert st == 0 and 0 <= cfg < lg.gemm_num_configs()
    assert lg.gemm_autotune_lookup(M, N, K, la, lb, F16, F32, F32) == cfg
    # D holds a correct result
    got = dp.result()
    ref = oracle_full(prob)
    compare(prob, region(prob, got), region(prob, ref), False, label="after autotune")
    tuned = _bits(dp)
    # gemm_run now runs the recorded entry: bit-identical to forcing it
    dp.reset_D()
    dp.run()
    assert np.array_equal(_bits(dp), tuned)
    dp.reset_D()
    dp.run(config=cfg)
    assert np.array_equal(_bits(dp), tuned)
    # after clearing, gemm_run is back on the static choice
    lg.gemm_autotune_clear()
    assert lg.gemm_autotune_lookup(M, N, K, la, lb, F16, F32, F32) == -1
    static = lg.gemm_select_config(M, N, K, la, lb, F16, F32, F32)
    dp.reset_D()
    dp.run()
    plain = _bits(dp)
    dp.reset_D()
    dp.run(config=static)
    assert np.array_equal(_bits(dp), plain)


def test_autotune_column_major_d_is_keyed_as_its_transpose():
    lg.gemm_autotune_clear()
    M, N, K = 600, 900, 256
    ep = W.make_epilogue_problem(M, N, K, layoutD=COL_MAJOR, values="int", c_values=None,
                                 bias_values="int", act=lg.GEMM_ACT_RELU, seed=6100)
    A = torch.from_numpy(ep.A.view(np.int16)).cuda()
    B = torch.from_numpy(ep.B.view(np.int16)).cuda()
    D = torch.from_numpy(ep.D).cuda()
    bias = torch.from_numpy(ep.bias).cuda()
    epi = lg.GemmEpilogue(ep.alpha, ep.beta, bias.data_ptr(), ep.act, ep.layoutC, ep.layoutD)
    s = torch.cuda.current_stream().cuda_stream
    st, cfg = lg.gemm_autotune(M, N, K, A.data_ptr(), ep.lda, ep.layoutA, B.data_ptr(), ep.ldb,
                               ep.layoutB, None, ep.ldc, D.data_ptr(), ep.ldd, F16, F32, F32, 0,
                               epi, 2, s)
    assert st == 0 and cfg >= 0
    assert lg.gemm_autotune_lookup(M, N, K, ROW_MAJOR, ROW_MAJOR, F16, F32, F32, COL_MAJOR) == cfg
    # the transposed signature (N x M, flipped layouts, row-major D) is the same key
    assert lg.gemm_autotune_lookup(N, M, K, COL_MAJOR, COL_MAJOR, F16, F32, F32, ROW_MAJOR) == cfg
    lg.gemm_autotune_clear()


def test_autotune_rejects_in_place():
    prob = W.make_problem(64, 64, 64, values="int", c_values="int", inplace=True, seed=6200)
    dp = DeviceProblem(prob)
    st, cfg = lg.gemm_autotune(*_args(dp), None, 2, torch.cuda.current_stream().cuda_stream)
    assert st == -6 and cfg == -1


@pytest.mark.parametrize("kind", ["i8", "fp8"])
def test_autotune_8_bit_inputs_stays_in_its_class(kind):
    """int8 and fp8 signatures only time the entries of their own class; the
    recorded entry then runs for gemm_run, and D is bit-exact against the
    oracle (integer-valued data)."""
    lg.gemm_autotune_clear()
    M, N, K = 700, 900, 512
    if kind == "i8":
        prob = W.make_int8_problem(M, N, K, values="full", c_values="int", seed=6300)
        prefix = "i8_"
    else:
        prob = W.make_problem(M, N, K, layoutA=ROW_MAJOR, layoutB=COL_MAJOR,
                              in_dtype=W.FP8_E4M3, values="int", c_values="int", seed=6301)
        prefix = "fp8_"
    log("case: autotune %s %dx%dx%d" % (kind, M, N, K))
    dp = DeviceProblem(prob)
    s = torch.cuda.current_stream().cuda_stream
    st, cfg = lg.gemm_autotune(*_args(dp), None, 2, s)
    assert st == 0 and lg.gemm_config_name(cfg).startswith(prefix)
    assert lg.gemm_autotune_lookup(M, N, K, prob.layoutA, prob.layoutB, prob.in_dtype,
                                   prob.acc_dtype, prob.out_dtype) == cfg
    got = dp.result()
    if kind == "i8":
        ref = prob.D.copy()
        oracle.gemm_i8(M, N, K, prob.A.ravel(), prob.lda, prob.layoutA, prob.B.ravel(),
                       prob.ldb, prob.layoutB, prob.C.ravel(), prob.ldc, ROW_MAJOR, ref.ravel(),
                       prob.ldd, ROW_MAJOR, prob.satf)
    else:
        ref = oracle_full(prob)
    assert np.array_equal(region(prob, got).view(np.uint8), region(prob, ref).view(np.uint8))
    dp.reset_D()
    dp.run()
    assert np.array_equal(dp.result().view(np.uint8), got.view(np.uint8))
    lg.gemm_autotune_clear()
