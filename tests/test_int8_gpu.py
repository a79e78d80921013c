"""GPU parity of int8 x int8 -> int32 (in_dtype GEMM_I8) through the C ABI
against the oracle's gemm_i8.  Integer results are compared bit for bit."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import dense_mixed_precision_tiled_amd as lg
import oracle
from dense_mixed_precision_tiled_amd import workloads as W
from dense_mixed_precision_tiled_amd.workloads import COL_MAJOR, F16, F32, ROW_MAJOR
from gpu_util import DeviceProblem, log, oracle_whole

pytestmark = pytest.mark.gpu

I8, I32 = lg.GEMM_I8, lg.GEMM_I32
# int8 tile-table entries -> block tile edge (None: skinny split-K)
I8_ENTRY_TILE = {5: 256, 6: 128, 7: 64, 8: None}


def _shape(cid):
    bm = I8_ENTRY_TILE[cid]
    return (13, 3 * 128 - 5, 2200) if bm is None else (2 * bm + 17, 3 * bm - 5, 400)


def oracle_i8(prob, layoutD=ROW_MAJOR):
    D = prob.D.copy()
    C = D if prob.inplace else prob.C
    oracle.gemm_i8(prob.M, prob.N, prob.K, prob.A.ravel(), prob.lda, prob.layoutA,
                   prob.B.ravel(), prob.ldb, prob.layoutB, None if C is None else C.ravel(),
                   prob.ldc, ROW_MAJOR, D.ravel(), prob.ldd, layoutD, prob.satf)
    return D


def _check(prob, config=None, label=""):
    log("case: %s config=%s" % (label, config))
    dp = DeviceProblem(prob)
    dp.run(config=config)
    got = dp.result()
    ref = oracle_i8(prob)
    bad = np.argwhere(got != ref)
    assert bad.size == 0, "%s: %d of %d differ, e.g. %s got %s ref %s" % (
        label, len(bad), got.size, bad[:3].tolist(), got[tuple(bad[:3].T)], ref[tuple(bad[:3].T)])


def test_int8_entries_are_in_the_table():
    for cid, bm in I8_ENTRY_TILE.items():
        name = lg.gemm_config_name(cid)
        assert name.startswith("i8_"), name
        if bm is not None:
            assert "_%dx%dx" % (bm, bm) in name, name
    assert lg.gemm_config_name(I8_DMA).startswith("i8_large_dma8_256x256x")
    assert lg.gemm_config_name(I8_DMA16).startswith("i8_large_dma_256x256x128_w2x2_mfma16x16x64")


@pytest.mark.parametrize("cid", sorted(I8_ENTRY_TILE))
@pytest.mark.parametrize("la,lb", [(ROW_MAJOR, COL_MAJOR), (ROW_MAJOR, ROW_MAJOR),
                                   (COL_MAJOR, COL_MAJOR), (COL_MAJOR, ROW_MAJOR)])
def test_every_int8_entry_and_layout(cid, la, lb):
    M, N, K = _shape(cid)
    prob = W.make_int8_problem(M, N, K, layoutA=la, layoutB=lb, values="full", c_values="big",
                               ldd=N + 3, seed=8000 + cid)
    _check(prob, cid, "i8 cfg%d A%d B%d" % (cid, la, lb))


def _ld16(x):
    """A leading dimension of whole 16-byte lines, one line past the extent."""
    return (x + 15) // 16 * 16 + 16


@pytest.mark.parametrize("cid", sorted(I8_ENTRY_TILE))
@pytest.mark.parametrize("la,lb", [(ROW_MAJOR, ROW_MAJOR), (COL_MAJOR, COL_MAJOR),
                                   (COL_MAJOR, ROW_MAJOR)])
@pytest.mark.parametrize("ragged", [True, False])
def test_m_or_n_contiguous_operands_on_the_vector_path(cid, la, lb, ragged):
    """16-byte aligned leading dimensions: row-major B and column-major A take
    the transposing 8-bit vector loads (dword loads along M or N, transposed
    in registers), with edge rows clamped, a ragged last K-tile masked, and
    the padding lines poisoned."""
    M, N, K = _shape(cid)
    # K + 3: a last K-tile that ends inside a 16-row block of the transposing
    # loader; 512: a whole number of K-tiles of every entry
    K = K + 3 if ragged else 512
    lda = _ld16(K if la == ROW_MAJOR else M)
    ldb = _ld16(N if lb == ROW_MAJOR else K)
    prob = W.make_int8_problem(M, N, K, layoutA=la, layoutB=lb, values="full", c_values="big",
                               lda=lda, ldb=ldb, ldd=N + 3, seed=8050 + cid + 3 * la + lb)
    _check(prob, cid, "i8 cfg%d A%d B%d K%d vector" % (cid, la, lb, K))


# the eight-wave LDS-DMA int8 entry: 16-byte aligned lines only (M- or
# N-contiguous operands take the transposing byte reads)
I8_DMA = 17


@pytest.mark.parametrize("la,lb", [(ROW_MAJOR, COL_MAJOR), (ROW_MAJOR, ROW_MAJOR),
                                   (COL_MAJOR, COL_MAJOR), (COL_MAJOR, ROW_MAJOR)])
@pytest.mark.parametrize("ragged", [True, False])
def test_dma_entry_every_layout(la, lb, ragged):
    """Ragged M and N, a ragged last K-tile (its k >= K part zeroed in LDS) or
    whole K-tiles, padding lines poisoned, C across the int32 range: wrapping
    with an odd ldd (staged epilogue), clamping (satf) with ldc = ldd a
    multiple of 4 (register epilogue on the interior tiles)."""
    M, N = 2 * 256 + 17, 3 * 256 - 5
    K = 403 if ragged else 512
    lda = _ld16(K if la == ROW_MAJOR else M)
    ldb = _ld16(N if lb == ROW_MAJOR else K)
    for satf in (0, 1):
        ld = (N + 3) // 4 * 4 + 4 if satf else N + 3
        prob = W.make_int8_problem(M, N, K, layoutA=la, layoutB=lb, values="full",
                                   c_values="big", satf=satf, lda=lda, ldb=ldb, ldc=ld, ldd=ld,
                                   seed=8800 + 2 * satf + ragged + 4 * la + 8 * lb)
        _check(prob, I8_DMA, "i8 dma A%d B%d K%d satf %d" % (la, lb, K, satf))


# the four-wave LDS-DMA int8 entry (16x16x64 MFMA): K-contiguous operands on
# 16-byte aligned lines only
I8_DMA16 = 19


@pytest.mark.parametrize("ragged", [True, False])
@pytest.mark.parametrize("satf", [0, 1])
def test_four_wave_dma_entry(ragged, satf):
    """Ragged M and N, a ragged last K-tile or whole K-tiles, padding lines
    poisoned, C across the int32 range: wrapping with an odd ldd (staged
    epilogue), clamping with ldc = ldd a multiple of 4 (register epilogue)."""
    M, N = 2 * 256 + 17, 3 * 256 - 5
    K = 403 if ragged else 512
    for inplace in (False, True):
        ld = (N + 3) // 4 * 4 + 4 if satf else N + 3
        prob = W.make_int8_problem(M, N, K, layoutA=ROW_MAJOR, layoutB=COL_MAJOR, values="full",
                                   c_values="big", satf=satf, inplace=inplace,
                                   lda=_ld16(K), ldb=_ld16(K), ldc=ld, ldd=ld,
                                   seed=8830 + 2 * satf + ragged + 4 * inplace)
        _check(prob, I8_DMA16, "i8 dma4 K%d satf %d inplace %d" % (K, satf, inplace))


def test_four_wave_dma_entry_rejects_other_operands():
    """M- or N-contiguous operands and unaligned lines: forced onto the
    entry, the call is rejected."""
    M, N, K = 100, 90, 160
    cases = [(ROW_MAJOR, ROW_MAJOR, K, _ld16(N)), (COL_MAJOR, COL_MAJOR, _ld16(M), K),
             (COL_MAJOR, ROW_MAJOR, _ld16(M), _ld16(N)), (ROW_MAJOR, COL_MAJOR, K + 1, K)]
    for la, lb, lda, ldb in cases:
        prob = W.make_int8_problem(M, N, K, layoutA=la, layoutB=lb, values="small", lda=lda,
                                   ldb=ldb, seed=8840)
        with pytest.raises(lg.GemmError) as e:
            DeviceProblem(prob).run(config=I8_DMA16)
        assert e.value.status == -8, (la, lb)


def test_dma_entry_in_place():
    prob = W.make_int8_problem(300, 700, 1000, layoutA=ROW_MAJOR, layoutB=ROW_MAJOR,
                               values="full", c_values="big", inplace=True, satf=1,
                               lda=_ld16(1000), ldb=_ld16(700), ldd=704, seed=8810)
    _check(prob, I8_DMA, "i8 dma in place")


def test_dma_entry_rejects_unaligned_lines():
    """Lines that are not whole 16-byte units are not this entry's: forced
    onto it, the call is rejected."""
    M, N, K = 100, 90, 160
    for la, lb, lda, ldb in ((ROW_MAJOR, COL_MAJOR, K + 1, K), (ROW_MAJOR, ROW_MAJOR, K, N + 3)):
        prob = W.make_int8_problem(M, N, K, layoutA=la, layoutB=lb, values="small", lda=lda,
                                   ldb=ldb, seed=8821)
        with pytest.raises(lg.GemmError) as e:
            DeviceProblem(prob).run(config=I8_DMA)
        assert e.value.status == -8


@pytest.mark.parametrize("cid", sorted(I8_ENTRY_TILE))
def test_satf_clamps_and_in_place(cid):
    M, N, K = _shape(cid)
    # C spans the whole int32 range, so C + A x B leaves it for some outputs
    prob = W.make_int8_problem(M, N, K, values="full", c_values="big", inplace=True, satf=1,
                               ldd=N + 1, seed=8100 + cid)
    _check(prob, cid, "i8 cfg%d satf in place" % cid)


@pytest.mark.parametrize("cid", sorted(I8_ENTRY_TILE))
@pytest.mark.parametrize("satf", [0, 1])
def test_vector_epilogue_with_c_near_the_int32_limits(cid, satf):
    """ldc = ldd a multiple of 4 (vector C and D): interior tiles add C in
    the register epilogue, edge tiles group by group; C spans the int32 range
    so C + A x B wraps (satf = 0) or clamps (satf = 1) for some outputs."""
    M, N, K = _shape(cid)
    ld = (N + 3) // 4 * 4 + 4
    prob = W.make_int8_problem(M, N, K, values="full", c_values="big", satf=satf, ldc=ld,
                               ldd=ld, seed=8150 + cid + 10 * satf)
    _check(prob, cid, "i8 cfg%d vector C satf %d" % (cid, satf))


@pytest.mark.parametrize("shape", [(1, 1, 1), (5, 7, 3), (33, 65, 129), (70, 45, 0),
                                   (64, 64, 4096 + 17)])
def test_small_and_ragged_shapes(shape):
    M, N, K = shape
    prob = W.make_int8_problem(M, N, K, values="full", c_values="int", seed=8200 + M)
    _check(prob, None, "i8 %dx%dx%d" % shape)


def test_unaligned_leading_dims_take_the_element_path():
    prob = W.make_int8_problem(100, 90, 300, lda=301, ldb=303, ldd=95, values="full",
                               c_values="int", seed=8300)
    _check(prob, None, "i8 unaligned")


def test_large_unaligned_operands_are_repacked():
    """M*N*K >= 2^30 with unaligned leading dimensions: the operands are
    copied into the workspace with 16-byte lines, then the vector path."""
    prob = W.make_int8_problem(1030, 1031, 1029, layoutB=ROW_MAJOR, lda=1029 + 3,
                               ldb=1031 + 5, values="full", c_values="big", ldd=1033,
                               seed=8310)
    _check(prob, None, "i8 repacked")


def test_wraps_modulo_2_32_beyond_2_17_products():
    """K = 140000 products of magnitude up to 2^14: sums leave the int32 range
    and wrap, exactly as the oracle's modular reduction of the exact sum."""
    M, N, K = 64, 64, 140000
    prob = W.make_int8_problem(M, N, K, values="full", c_values=None, seed=8400)
    # push sums past 2^31: most rows all +127 or -128
    prob.A[:, :K] = np.where(np.arange(M)[:, None] % 3 == 0, -128, 127).astype(np.int8)
    prob.B[:, :K] = np.int8(127)
    ref = oracle_i8(prob)
    exact = [int(np.int64(K) * int(prob.A[i, 0]) * 127) for i in range(M)]
    assert any(abs(e) > 2 ** 31 for e in exact)
    _check(prob, None, "i8 wrap")


def test_satf_with_k_at_or_above_2_17_is_rejected():
    prob = W.make_int8_problem(8, 8, 1 << 17, values="small", satf=1, seed=8500)
    dp = DeviceProblem(prob)
    with pytest.raises(lg.GemmError) as e:
        dp.run()
    assert e.value.status == -4


def test_column_major_d_and_rejected_epilogues():
    M, N, K = 300, 200, 256
    prob = W.make_int8_problem(M, N, K, values="full", c_values=None, seed=8600)
    dp = DeviceProblem(prob)
    Dc = torch.full((N, M), 7, dtype=torch.int32, device="cuda")
    s = torch.cuda.current_stream().cuda_stream
    args = (M, N, K, dp.A.data_ptr(), prob.lda, prob.layoutA, dp.B.data_ptr(), prob.ldb,
            prob.layoutB, None, prob.ldc, Dc.data_ptr(), M, I8, I32, I32, 0)
    assert lg.gemm_run_ex(*args, lg.GemmEpilogue(layoutD=COL_MAJOR), s) == 0
    torch.cuda.synchronize()
    ref = np.zeros(N * M, dtype=np.int32)
    oracle.gemm_i8(M, N, K, prob.A.ravel(), prob.lda, prob.layoutA, prob.B.ravel(), prob.ldb,
                   prob.layoutB, None, N, ROW_MAJOR, ref, M, COL_MAJOR, 0)
    assert np.array_equal(Dc.cpu().numpy().ravel(), ref)
    for epi in (lg.GemmEpilogue(alpha=2.0), lg.GemmEpilogue(activation=lg.GEMM_ACT_RELU)):
        assert lg.gemm_run_ex(*args, epi, s) == -4


def test_config_class_mismatch_is_rejected():
    prob = W.make_int8_problem(64, 64, 64, values="small", seed=8700)
    dp = DeviceProblem(prob)
    with pytest.raises(lg.GemmError) as e:
        dp.run(config=0)          # a 16-bit entry
    assert e.value.status == -8
    f16 = W.make_problem(64, 64, 64, values="int", seed=8701)
    with pytest.raises(lg.GemmError) as e:
        DeviceProblem(f16).run(config=5)   # an int8 entry
    assert e.value.status == -8


def test_multi_round_ragged_row_order_raster():
    """17 x 19 tiles of 256 with K <= 2048 (plain row-order tile walk), int32
    C: the whole output bit for bit against the oracle's product form."""
    M, N, K = 4100, 4610, 1000
    prob = W.make_int8_problem(M, N, K, values="full", c_values="int", seed=8900)
    log("case: i8 %dx%dx%d (whole output)" % (M, N, K))
    dp = DeviceProblem(prob)
    dp.run()
    got = dp.result()
    assert np.array_equal(got, oracle_whole(prob))


def test_4096_int8_whole_output():
    """The int8 workload the benchmark times: 4096^3, A row-major, B
    column-major, int32 D; every output against the oracle's product form
    (exact integer sums), bit for bit."""
    n = 4096
    prob = W.make_int8_problem(n, n, n, values="full", c_values=None, seed=8800)
    log("case: i8 4096^3 (whole output)")
    dp = DeviceProblem(prob)
    dp.run()
    got = dp.result()
    ref = oracle_whole(prob)
    assert np.array_equal(got, ref)
