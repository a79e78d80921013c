"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Every output element is compared: small shapes against the per-element
oracle, the full-size workloads against the oracle's product form (fp64
library matmul of the exactly decoded operands, then the oracle's epilogue
and single rounding).  Integer-valued inputs must be bit-exact; random inputs
meet the tolerances stated in gpu_util, the relative Frobenius bar over all
M x N outputs.
"""
import numpy as np
import pytest
import torch

import dense_mixed_precision_tiled_amd as lg
import oracle
from dense_mixed_precision_tiled_amd import workloads as W
from dense_mixed_precision_tiled_amd.workloads import BF16, COL_MAJOR, F16, F32, ROW_MAJOR
from gpu_util import (DeviceProblem, check_padding, compare, log, oracle_full, oracle_whole,
                      product_sums, region)

pytestmark = pytest.mark.gpu

@pytest.fixture(scope="module", autouse=True)
def device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    lg.library()  # raises if the HIP library is missing: no fallback
    torch.cuda.init()
    yield


def _full_check(prob, exact, config=None, label=None):
    label = label or prob.name
    log("case: %s config=%s" % (label, config))
    dp = DeviceProblem(prob)
    dp.run(config=config)
    got = dp.result()
    ref = oracle_full(prob)
    compare(prob, region(prob, got), region(prob, ref), exact, label=label)
    check_padding(prob, got, label)
    return got


def _whole_check(prob, exact, label=None, sums=None):
    """The whole M x N output against the oracle's product form."""
    label = label or prob.name
    log("case: %s (whole output)" % label)
    dp = DeviceProblem(prob)
    dp.run()
    got = dp.result()
    ref = oracle_whole(prob, sums=sums)
    compare(prob, region(prob, got), region(prob, ref), exact, label=label)
    check_padding(prob, got, label)
    return got


# ------------------------------------------------------------ the workloads

@pytest.mark.parametrize("values,exact", [("uniform", False), ("int", True)])
def test_256_cube(values, exact):
    _full_check(W.w_256(values), exact)


@pytest.mark.parametrize("values,exact", [("uniform", False), ("int", True)])
def test_4096_fp16_to_fp32(values, exact):
    _whole_check(W.w_4096_f16(values), exact)


@pytest.mark.parametrize("values,exact", [("normal", False), ("int", True)])
def test_4096_bf16_colB_inplace(values, exact):
    # integer variant: integer A and B, C normal(0,1); fl32(S + C) with S exact
    # equals the oracle's single rounding of S + C
    _whole_check(W.w_4096_bf16_inplace(values), exact)


@pytest.mark.parametrize("values,exact", [("uniform", False), ("int", True)])
def test_hgemm_ragged_overflow(values, exact):
    """Both satf modes over the whole 3999 x 4001 output (one set of oracle
    sums for the two)."""
    sums = None
    for satf in (0, 1):
        prob = W.w_hgemm(satf, values)
        assert len(prob.extra["scaled_rows"]) == 40
        if sums is None:
            sums = product_sums(prob)
        D = _whole_check(prob, exact, label="%s satf=%d" % (prob.name, satf), sums=sums)
        v = W.from_bits16(D[:prob.M, :prob.N], F16)
        if satf:
            assert np.isfinite(v).all(), "satf left a non-finite value"
        else:
            assert np.isinf(v).any(), "the scaled rows should overflow fp16"


@pytest.mark.parametrize("values,exact", [("uniform", False), ("int", True)])
def test_wide_16384x16384x1024(values, exact):
    _whole_check(W.w_wide(values), exact)


@pytest.mark.parametrize("values,exact", [("uniform", False), ("int", True)])
def test_skinny_16x16384x16384(values, exact):
    _whole_check(W.w_skinny(values), exact)


@pytest.mark.parametrize("values,exact", [("uniform", False), ("int", True)])
def test_multi_round_ragged_skewed_raster(values, exact):
    """17 x 19 tiles of 256 (more than one per CU) with K <= 2048: the host
    walks the tiles in groups of 2 tile-rows with staggered starting columns
    (the last group holds one tile-row) instead of groups of 4.  Ragged M and
    N, fp32 C; the whole output."""
    prob = W.make_problem(4100, 4610, 1000, values=values, c_values="normal" if values ==
                          "uniform" else "int", seed=20311, name="4100x4610x1000 +C")
    _whole_check(prob, exact)


def test_operand_past_the_32_bit_byte_range():
    """A of 65600 x 32768 fp16 (4.3 GB) lies past the byte range that the
    buffer loads' 32-bit offsets address: the call takes the element-wise
    loads (64-bit offsets; the operand copy for alignment would be as large,
    so none is made) and must stay exact.  Integer-valued data from
    pattern_int; rows on both sides of the 4 GiB mark, the first and the last
    rows compared bit for bit with the oracle."""
    M, K, N = 65600, 32768, 48
    assert M * K * 2 > (1 << 32)
    log("case: A past 4 GiB, %dx%dx%d" % (M, N, K))
    dev = torch.device("cuda")
    A = torch.empty(M, K, dtype=torch.float16, device=dev)
    kk = torch.arange(K, device=dev, dtype=torch.int64)[None, :]
    for r0 in range(0, M, 4096):
        rr = torch.arange(r0, min(M, r0 + 4096), device=dev, dtype=torch.int64)[:, None]
        A[r0:r0 + rr.shape[0]] = W.pattern_int(rr, kk).to(torch.float16)
    kb, nb = np.arange(K)[:, None], np.arange(N)[None, :]
    Bh = W.pattern_int(kb + 3, nb).astype(np.float16)
    B = torch.from_numpy(Bh).to(dev)
    D = torch.full((M, N), float("nan"), dtype=torch.float32, device=dev)
    st = lg.gemm_run(M, N, K, A.data_ptr(), K, ROW_MAJOR, B.data_ptr(), N, ROW_MAJOR, None, N,
                     D.data_ptr(), N, F16, F32, F32, 0, torch.cuda.current_stream().cuda_stream)
    assert st == 0, lg.gemm_status_string(st)
    rows = np.array([0, 1, 32767, 32768, 65535, 65536, 65537, M - 2, M - 1])
    got = D[torch.from_numpy(rows).to(dev)].cpu().numpy()
    del A, D
    As = W.pattern_int(rows[:, None], np.arange(K)[None, :]).astype(np.float16)
    ref = np.zeros((len(rows), N), np.float32)
    oracle.gemm(len(rows), N, K, As.view(np.uint16).ravel(), K, ROW_MAJOR,
                Bh.view(np.uint16).ravel(), N, ROW_MAJOR, None, N, ref.ravel(), N,
                F16, F32, F32, 0)
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))


# ------------------------------------------------- every tile-table entry

# tile-table entries: id -> block tile edge (None: the skinny split-K entry);
# test_config_ids_match_table checks this against the library's table
ENTRY_TILE = {0: 256, 1: 128, 2: 64, 3: None, 4: 256, 13: 256, 14: 32, 15: 256, 16: 256}
# entries whose kernels load 16-byte aligned operands only (LDS DMA): their
# sweeps use leading dimensions rounded up to 8 elements (still ragged M, N
# and K, padding poisoned with NaN)
VEC_ONLY = {13, 15, 16}


def _align(cid):
    return 8 if cid in VEC_ONLY else 1


def _entry_shapes():
    out = []
    for cid, bm in ENTRY_TILE.items():
        if bm is None:
            out.append((cid, 13, 3 * 128 - 5, 1100))
        else:
            out.append((cid, 2 * bm + 17, 3 * bm - 5, 200))
    return out


def _bits16(x: np.ndarray, in_dtype: int) -> np.ndarray:
    """fp16 or bf16 bit patterns of values exact in both formats."""
    if in_dtype == F16:
        return x.astype(np.float16).view(np.uint16)
    return (x.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)


@pytest.mark.parametrize("in_dtype", [F16, BF16])
@pytest.mark.parametrize("K", [64, 256])
def test_f16_products_far_below_the_largest_are_kept(K, in_dtype):
    """Unlike the fp8 MFMA (test_fp8_gpu.test_fp8_group_truncation), the
    16-bit MFMAs keep products far below the largest one: A holds 2^8 at
    every k % 64 == 0 and 2^(8-r) elsewhere, B holds 2^8, so each row sums
    one product 2^16 and 63 products 2^(16-r) per 64 k; for r up to 22 the
    sum is representable in fp32, and every 16-bit entry returns it exactly."""
    M, N = 64, 64
    for r in (14, 18, 22):
        prob = W.make_problem(M, N, K, layoutA=ROW_MAJOR, layoutB=COL_MAJOR, values="int",
                              in_dtype=in_dtype, seed=9950)
        a = np.full((M, K), 2.0 ** (8 - r))
        a[:, 0:K:64] = 256.0
        prob.A[:, :K] = _bits16(a, in_dtype)
        prob.B[:, :K] = _bits16(np.full((N, K), 256.0), in_dtype)
        exact = (K // 64) * (2.0 ** 16 + 63 * 2.0 ** (16 - r))
        assert np.all(region(prob, oracle_full(prob)).astype(np.float64) == exact)
        for cid in sorted(ENTRY_TILE):
            log("case: 16-bit small products dtype %d r %d K %d config %d" % (in_dtype, r, K, cid))
            dp = DeviceProblem(prob)
            dp.run(config=cid)
            got = region(prob, dp.result()).astype(np.float64)
            assert np.all(got == exact), (cid, r, got.ravel()[:4], exact)


def test_config_ids_match_table():
    # 16-bit entries here; the int8 entries (ids 5..8, 17, 19) and the fp8
    # entries (ids 9..12, 18) are covered by test_int8_gpu and test_fp8_gpu
    assert lg.gemm_num_configs() == len(ENTRY_TILE) + 11
    assert lg.gemm_config_name(17).startswith("i8_")
    assert lg.gemm_config_name(18).startswith("fp8_")
    assert lg.gemm_config_name(19).startswith("i8_")
    assert lg.gemm_config_name(13).startswith("large_dma")
    for cid in range(5, 9):
        assert lg.gemm_config_name(cid).startswith("i8_")
    for cid in range(9, 13):
        assert lg.gemm_config_name(cid).startswith("fp8_")
    for cid, bm in ENTRY_TILE.items():
        name = lg.gemm_config_name(cid)
        if bm is None:
            assert name.startswith("skinny"), name
        else:
            assert "_%dx%dx" % (bm, bm) in name, name


@pytest.mark.parametrize("cid,M,N,K", _entry_shapes())
def test_every_entry_layouts_dtypes(cid, M, N, K):
    for in_dt in (F16, BF16):
        for la in (ROW_MAJOR, COL_MAJOR):
            for lb in (ROW_MAJOR, COL_MAJOR):
                for values, exact in (("int", True), ("uniform", False)):
                    prob = W.make_problem(M, N, K, layoutA=la, layoutB=lb, in_dtype=in_dt,
                                          values=values, seed=1000 + cid, align=_align(cid))
                    _full_check(prob, exact, config=cid,
                                label="cfg%d %dx%dx%d in=%d A%d B%d %s" % (
                                    cid, M, N, K, in_dt, la, lb, values))


@pytest.mark.parametrize("cid,M,N,K", _entry_shapes())
def test_every_entry_output_modes(cid, M, N, K):
    modes = [
        dict(out_dtype=F16, acc_dtype=F16, c_values="uniform", ldd=N + 3, satf=1),
        dict(out_dtype=BF16, acc_dtype=F32, c_values="normal", ldd=N + 8),
        dict(out_dtype=F32, acc_dtype=F32, c_values="normal", inplace=True, ldd=N + 5),
        dict(out_dtype=F32, acc_dtype=F32, c_values=None, lda=None, ldd=N + 1),
    ]
    for mode in modes:
        for values, exact in (("int", True), ("uniform", False)):
            cv = mode.get("c_values")
            if values == "int" and cv is not None:
                mode = dict(mode, c_values="int")
            prob = W.make_problem(M, N, K, layoutA=ROW_MAJOR, layoutB=COL_MAJOR,
                                  in_dtype=F16, values=values, seed=2000 + cid,
                                  align=_align(cid), **mode)
            _full_check(prob, exact, config=cid,
                        label="cfg%d out=%d acc=%d inplace=%s %s" % (
                            cid, prob.out_dtype, prob.acc_dtype, prob.inplace, values))


@pytest.mark.parametrize("cid", sorted(ENTRY_TILE))
@pytest.mark.parametrize("out_dt,acc_dt", [(F16, F16), (BF16, F32), (F32, F32)])
def test_every_entry_c_on_the_vector_epilogue(cid, out_dt, acc_dt):
    """Nonzero C with ldc = ldd a multiple of 4 (C and D vector-friendly):
    interior tiles add C in the register epilogue, edge tiles in the staged
    pre-phase (their groups crossing column N element by element).  Ragged M
    and N (N % 4 = 3)."""
    M, N, K = next((m, n, k) for c, m, n, k in _entry_shapes() if c == cid)
    ld = (N + 3) // 4 * 4 + 4
    for values, exact in (("int", True), ("uniform", False)):
        prob = W.make_problem(M, N, K, layoutA=ROW_MAJOR, layoutB=ROW_MAJOR, in_dtype=F16,
                              acc_dtype=acc_dt, out_dtype=out_dt, values=values,
                              c_values="int" if exact else "normal", ldc=ld, ldd=ld,
                              seed=2100 + cid, align=_align(cid))
        _full_check(prob, exact, config=cid,
                    label="cfg%d vector C out=%d %s" % (cid, out_dt, values))


@pytest.mark.parametrize("cid", sorted(ENTRY_TILE))
def test_unaligned_leading_dims(cid):
    # lda, ldb not multiples of 8 elements: the element-wise load path (an
    # LDS-DMA entry forced on them is rejected; the dispatcher's choice for
    # a large unaligned problem falls back to register-staged loads)
    M, N, K = (37, 45, 77) if ENTRY_TILE[cid] is not None else (9, 300, 700)
    for la, lb in ((ROW_MAJOR, ROW_MAJOR), (COL_MAJOR, COL_MAJOR)):
        a_in = K if la == ROW_MAJOR else M
        b_in = N if lb == ROW_MAJOR else K
        prob = W.make_problem(M, N, K, layoutA=la, layoutB=lb, values="int",
                              lda=a_in + 1, ldb=b_in + 3, ldd=N + 2, c_values="int",
                              seed=3000 + cid)
        if cid in VEC_ONLY:
            with pytest.raises(lg.GemmError) as e:
                DeviceProblem(prob).run(config=cid)
            assert e.value.status == -8
            continue
        _full_check(prob, True, config=cid, label="cfg%d unaligned A%d B%d" % (cid, la, lb))


@pytest.mark.parametrize("values,exact", [("int", True), ("uniform", False)])
def test_large_unaligned_falls_back_to_staged_loads(values, exact):
    """A large problem with unaligned lda / ldb: the dispatcher picks the
    large tile, whose LDS-DMA kernel cannot take these operands; the
    register-staged large tile runs it (ragged M, N, K; fp32 C)."""
    prob = W.make_problem(1030, 777, 301, values=values, lda=301 + 3, ldb=777 + 1,
                          c_values="int" if exact else "normal", ldd=781, seed=3100)
    _full_check(prob, exact, label="large unaligned %s" % values)


@pytest.mark.parametrize("la,lb", [(ROW_MAJOR, ROW_MAJOR), (ROW_MAJOR, COL_MAJOR),
                                   (COL_MAJOR, ROW_MAJOR), (COL_MAJOR, COL_MAJOR)])
def test_large_unaligned_operands_are_repacked(la, lb):
    """M*N*K >= 2^30 with leading dimensions that miss 16-byte lines: the
    library copies the operands into its workspace with aligned lines and
    runs the vector path (padding of the originals poisoned with NaN; ragged
    M, N and K; fp32 C).  Whole output against the oracle."""
    M, N, K = 1030, 1031, 1029
    lda = (K if la == ROW_MAJOR else M) + 3
    ldb = (N if lb == ROW_MAJOR else K) + 1
    for values, exact in (("int", True), ("uniform", False)):
        prob = W.make_problem(M, N, K, layoutA=la, layoutB=lb, values=values, lda=lda, ldb=ldb,
                              c_values="int" if exact else "normal", ldd=N + 2,
                              seed=3150 + 2 * la + lb)
        _full_check(prob, exact, label="repacked A%d B%d %s" % (la, lb, values))


@pytest.mark.parametrize("shape", [(1, 1, 1), (1, 7, 3), (5, 1, 9), (17, 33, 8), (31, 15, 9),
                                   (64, 64, 64), (65, 63, 65), (16, 16, 1), (33, 257, 31),
                                   (100, 100, 0)])
def test_small_and_degenerate_shapes(shape):
    M, N, K = shape
    for values, exact in (("int", True), ("uniform", False)):
        prob = W.make_problem(M, N, K, values=values, c_values="int" if exact else "normal",
                              ldd=N + 1, seed=4000 + M + N + K)
        _full_check(prob, exact, label="%dx%dx%d %s" % (M, N, K, values))


def test_empty_problem_writes_nothing():
    prob = W.make_problem(0, 8, 8, ldd=8)
    dp = DeviceProblem(prob)
    dp.run()
    prob2 = W.make_problem(8, 0, 8, ldd=1)
    dp2 = DeviceProblem(prob2)
    dp2.run()
    assert np.array_equal(dp2.result().view(np.uint8), prob2.D.view(np.uint8))


@pytest.mark.parametrize("out_dt", [F32, F16, BF16])
def test_satf_special_values_on_gpu(out_dt):
    """C = +Inf, -Inf, NaN with finite A*B -> +MAX_NORM, -MAX_NORM, +0 under
    satf; unchanged specials without it."""
    M, N, K = 40, 70, 33
    acc = F16 if out_dt == F16 else F32
    for satf in (0, 1):
        prob = W.make_problem(M, N, K, in_dtype=F16, acc_dtype=acc, out_dtype=out_dt,
                              values="int", c_values="int", satf=satf, seed=5000)
        specials = np.array([np.inf, -np.inf, np.nan], dtype=np.float32)
        C = W.from_bits16(prob.C, out_dt) if out_dt != F32 else prob.C.copy()
        C[::3, :N] = specials[0]
        C[1::3, :N] = specials[1]
        C[2::7, :N] = specials[2]
        prob.C = C if out_dt == F32 else W.to_bits16(C, out_dt)
        got = _full_check(prob, True, label="satf=%d out=%d" % (satf, out_dt))
        v = W.from_bits16(region(prob, got), out_dt) if out_dt != F32 else region(prob, got)
        if satf:
            assert np.isfinite(v).all()
        else:
            assert np.isinf(v).any() and np.isnan(v).any()


def test_golden_2x3_example_on_gpu():
    """The pages' 2x3 matrix stored col-major as A, times I3: D row-major is
    1,2,3,4,5,6 (the row-major order printed on the page)."""
    A = np.array([1, 4, 2, 5, 3, 6], dtype=np.float16).view(np.uint16).reshape(3, 2)
    B = np.eye(3, dtype=np.float16).view(np.uint16)
    prob = W.make_problem(2, 3, 3, layoutA=COL_MAJOR, values="zero", seed=1)
    prob.A = A.copy()
    prob.lda = 2
    prob.B = B.copy()
    dp = DeviceProblem(prob)
    dp.run()
    got = dp.result()
    assert list(got[:2, :3].ravel()) == [1, 2, 3, 4, 5, 6]


def test_nondefault_stream_and_determinism():
    prob = W.make_problem(300, 500, 700, values="uniform", seed=6000)
    dp = DeviceProblem(prob)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        dp.run(stream=s)
    s.synchronize()
    first = dp.result().copy()
    ref = oracle_full(prob)
    compare(prob, region(prob, first), region(prob, ref), False, label="side stream")
    for _ in range(3):
        dp.reset_D()
        dp.run()
        again = dp.result()
        assert np.array_equal(first.view(np.uint8), again.view(np.uint8)), "nondeterministic"


def test_two_threads_one_stream_growing_workspace():
    """Split-K calls (M <= 16) from two host threads on one stream, the second
    thread's problem growing every round so the library's workspace grows
    while the first thread's call may be between taking the buffer and
    launching.  The workspace lock keeps each call's slice and reduction
    launches together, and an outgrown buffer is never freed, so every
    result stays exact."""
    import threading

    s = torch.cuda.Stream()
    fixed = W.make_problem(16, 2048, 8192, values="int", seed=6100, name="fixed")
    growing = [W.make_problem(16, 1024 * (r + 1), 8192, values="int", seed=6110 + r,
                              name="grow%d" % r) for r in range(6)]
    log("case: two threads, one stream, growing workspace")
    dfix = [DeviceProblem(fixed) for _ in growing]
    dgrow = [DeviceProblem(p) for p in growing]
    torch.cuda.synchronize()
    start = threading.Barrier(2)
    errors = []

    def worker(devs):
        try:
            for d in devs:
                start.wait()
                d.run(stream=s)
        except Exception as e:  # reported below
            errors.append(e)

    t1 = threading.Thread(target=worker, args=(dfix,))
    t2 = threading.Thread(target=worker, args=(dgrow,))
    t1.start(), t2.start()
    t1.join(), t2.join()
    assert not errors, errors
    s.synchronize()
    ref_fixed = oracle_whole(fixed)
    for d in dfix:
        assert np.array_equal(d.result(), ref_fixed)
    for d, p in zip(dgrow, growing):
        assert np.array_equal(d.result(), oracle_whole(p)), p.name
