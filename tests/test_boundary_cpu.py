"""The C-ABI library on the host: it loads, exports every symbol the header
declares, and rejects bad arguments before any HIP call (no GPU needed)."""
import ctypes
import os
import re

import pytest

import dense_mixed_precision_tiled_amd as lg

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "libgemm.h")

R, Cm = lg.GEMM_ROW_MAJOR, lg.GEMM_COL_MAJOR
F32, F16, BF16 = lg.GEMM_F32, lg.GEMM_F16, lg.GEMM_BF16


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gemm_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(lg.LIB_PATH):
        from dense_mixed_precision_tiled_amd import build
        build.build()
    return lg.library()


def test_header_declares_the_calls():
    assert _declared_functions() == sorted(lg.SIGNATURES)


def test_every_declared_symbol_is_exported(lib):
    for name in _declared_functions():
        assert hasattr(lib, name), name


def test_status_strings(lib):
    for code in range(-9, 1):
        s = lg.gemm_status_string(code)
        assert s and s != "unknown status", code
    assert lg.gemm_status_string(-99) == "unknown status"


def test_config_table(lib):
    n = lg.gemm_num_configs()
    assert n >= 4
    names = [lg.gemm_config_name(i) for i in range(n)]
    assert all(names) and len(set(names)) == n
    assert lg.gemm_config_name(n) is None and lg.gemm_config_name(-1) is None


def test_dispatcher_shape_classes(lib):
    names = {i: lg.gemm_config_name(i) for i in range(lg.gemm_num_configs())}
    pick = lambda M, N, K: names[lg.gemm_select_config(M, N, K, R, R, F16, F32, F32)]
    assert pick(4096, 4096, 4096).startswith("large")
    assert pick(3999, 4001, 4104).startswith("large")
    assert pick(16384, 16384, 1024).startswith("large")
    # both operands K-contiguous (A row-major, B column-major): the LDS-DMA
    # tile with the 16x16x32 MFMA
    assert names[lg.gemm_select_config(4096, 4096, 4096, R, Cm, F16, F32, F32)] == \
        "large_dma_256x256x64_w2x2_mfma16x16x32"
    assert names[lg.gemm_select_config(4096, 4096, 4096, Cm, R, F16, F32, F32)].startswith("large8")
    assert pick(16, 16384, 16384).startswith("skinny")
    assert pick(256, 256, 256).startswith("tiny")     # 16 small tiles: 64 tiny ones
    assert pick(1024, 1024, 1024).startswith("small")
    I8, I32 = lg.GEMM_I8, lg.GEMM_I32
    pick8 = lambda M, N, K: names[lg.gemm_select_config(M, N, K, R, Cm, I8, I32, I32)]
    # int8: K-contiguous, aligned, whole K-tiles -> the four-wave LDS-DMA
    # tile; a ragged K or another layout -> the eight-wave register-staged one
    assert pick8(4096, 4096, 4096) == "i8_large_dma_256x256x128_w2x2_mfma16x16x64"
    assert pick8(4096, 4096, 4100).startswith("i8_large8")
    assert names[lg.gemm_select_config(4096, 4096, 4096, R, R, I8, I32, I32)].startswith(
        "i8_large8")
    assert pick8(16, 16384, 16384).startswith("i8_skinny")
    assert pick8(256, 256, 256).startswith("i8_small")
    # fp8: the eight-wave LDS-DMA tile in every layout (aligned operands)
    E4 = lg.GEMM_FP8_E4M3
    for la, lb in ((R, Cm), (R, R), (Cm, Cm), (Cm, R)):
        for K in (4096, 4100):
            assert names[lg.gemm_select_config(4096, 4096, K, la, lb, E4, F32, F32)] == \
                "fp8_large_dma8_256x256x128_w2x4_mfma32x32x64"
    assert lg.gemm_select_config(-1, 4, 4, R, R, F16, F32, F32) == -1
    assert lg.gemm_select_config(4, 4, 4, 7, R, F16, F32, F32) == -5
    assert lg.gemm_select_config(4, 4, 4, R, R, F32, F32, F32) == -4


# fake, distinct, 16-byte aligned addresses: gemm_validate never dereferences
A0, B0, C0, D0 = 0x10000000, 0x20000000, 0x30000000, 0x40000000


def v(M=8, N=8, K=8, A=A0, lda=None, la=R, B=B0, ldb=None, lb=R, C=None, ldc=None, D=D0,
      ldd=None, i=F16, a=F32, o=F32):
    lda = max(1, K if la == R else M) if lda is None else lda
    ldb = max(1, N if lb == R else K) if ldb is None else ldb
    ldd = max(1, N) if ldd is None else ldd
    ldc = max(1, N) if ldc is None else ldc
    return lg.gemm_validate(M, N, K, A, lda, la, B, ldb, lb, C, ldc, D, ldd, i, a, o)


def test_validation_ok_cases(lib):
    assert v() == 0
    assert v(la=Cm, lb=Cm) == 0
    assert v(C=C0) == 0
    assert v(C=D0) == 0                      # in place, ldc == ldd
    assert v(i=BF16, o=BF16) == 0
    assert v(i=F16, a=F16, o=F16) == 0       # HGEMM
    assert v(M=0, A=None, B=None, D=None) == 0
    assert v(N=0, A=None, B=None, D=None) == 0
    assert v(K=0, A=None, B=None, lda=1, ldb=8) == 0   # K = 0: A, B unused
    assert v(lda=13, ldb=9, ldd=11) == 0     # padded (unaligned) leading dims
    I8, I32 = lg.GEMM_I8, lg.GEMM_I32
    assert v(i=I8, a=I32, o=I32) == 0        # int8 x int8 -> int32
    assert v(i=I8, a=I32, o=I32, C=C0, la=Cm, lb=R) == 0


def test_validation_errors(lib):
    assert v(M=-1) == -1 and v(N=-1) == -1 and v(K=-1) == -1
    assert v(M=2 ** 31) == -1
    assert v(lda=7) == -2 and v(ldb=7) == -2 and v(ldd=7) == -2
    assert v(C=C0, ldc=7) == -2
    assert v(la=Cm, lda=7) == -2 and v(lb=Cm, ldb=7) == -2
    assert v(M=0, lda=0) == -2               # ld >= 1 always
    assert v(A=None) == -3 and v(B=None) == -3 and v(D=None) == -3
    assert v(i=F32) == -4 and v(a=BF16) == -4
    assert v(i=BF16, a=F16, o=F16) == -4 and v(a=F16, o=F32) == -4
    assert v(la=2) == -5 and v(lb=-1) == -5
    I8, I32 = lg.GEMM_I8, lg.GEMM_I32
    assert v(i=I8, a=F32, o=F32) == -4 and v(i=I8, a=I32, o=F32) == -4
    assert v(i=F16, a=I32, o=I32) == -4 and v(i=F16, a=F32, o=I32) == -4
    assert v(D=A0 + 64) == -6                # D inside A
    assert v(D=B0) == -6
    assert v(C=D0 + 4) == -6                 # C partially overlaps D
    assert v(C=D0, ldc=9, ldd=8) == -6       # same base, different ld


def vx(M=8, N=6, K=8, C=None, ldc=None, D=D0, ldd=None, alpha=1.0, beta=1.0, bias=0,
       act=0, lc=R, ld=R, o=F32):
    ldd = (N if ld == R else M) if ldd is None else ldd
    ldc = (N if lc == R else M) if ldc is None else ldc
    epi = lg.GemmEpilogue(alpha, beta, bias, act, lc, ld)
    return lg.gemm_validate_ex(M, N, K, A0, K, R, B0, N, R, C, ldc, D, ldd, F16, F32, o, epi)


def test_validation_ex_ok_cases(lib):
    assert vx() == 0
    assert lg.gemm_validate_ex(8, 8, 8, A0, 8, R, B0, 8, R, None, 8, D0, 8, F16, F32, F32,
                               None) == 0          # NULL epilogue = gemm_run
    assert vx(act=lg.GEMM_ACT_RELU) == 0 and vx(act=lg.GEMM_ACT_GELU) == 0
    assert vx(ld=Cm) == 0 and vx(C=C0, lc=Cm) == 0 and vx(C=C0, lc=Cm, ld=Cm) == 0
    assert vx(bias=0x50000000, alpha=0.5, beta=-2.0) == 0
    assert vx(C=D0, lc=Cm, ld=Cm) == 0             # in place, column-major
    assert vx(C=C0, ldc=1, beta=0.0) == 0          # beta == 0: C is not read
    assert vx(M=8, N=6, ld=Cm, ldd=8) == 0         # column-major D: ldd >= M


def test_validation_ex_errors(lib):
    assert vx(act=3) == -4 and vx(act=-1) == -4
    assert vx(lc=2) == -5 and vx(ld=7) == -5
    assert vx(ld=Cm, ldd=7) == -2                  # column-major D needs ldd >= M = 8
    assert vx(C=C0, lc=Cm, ldc=7) == -2            # column-major C needs ldc >= M
    assert vx(ld=R, ldd=5) == -2
    assert vx(bias=D0 + 8) == -6                   # bias inside D
    assert vx(C=D0, lc=R, ld=Cm, ldc=8, ldd=8) == -6   # same buffer, different layouts
    st = lg.gemm_run_ex(8, 6, 8, A0, 8, R, B0, 6, R, None, 6, D0, 6, F16, F32, F32, 0,
                        lg.GemmEpilogue(activation=9), None)
    assert st == -4                                # rejected before any HIP call


def test_autotune_host_side(lib):
    # argument errors come back before any HIP call; the cache starts empty
    st, cfg = lg.gemm_autotune(-1, 8, 8, A0, 8, R, B0, 8, R, None, 8, D0, 8, F16, F32, F32, 0,
                               None, 3, None)
    assert st == -1 and cfg == -1
    st, _ = lg.gemm_autotune(8, 8, 8, A0, 8, R, B0, 8, R, D0, 8, D0, 8, F16, F32, F32, 0,
                             None, 3, None)
    assert st == -6                          # in place: every candidate would apply it
    st, cfg = lg.gemm_autotune(0, 8, 8, A0, 8, R, B0, 8, R, None, 8, D0, 8, F16, F32, F32, 0,
                               None, 3, None)
    assert st == 0 and cfg == -1             # empty problem: nothing to tune
    lg.gemm_autotune_clear()
    assert lg.gemm_autotune_lookup(64, 64, 64, R, R, F16, F32, F32) == -1


def test_run_rejects_before_touching_the_device(lib):
    # argument errors return before any HIP call, so this works without a GPU
    st = lg.gemm_run(-1, 8, 8, A0, 8, R, B0, 8, R, None, 8, D0, 8, F16, F32, F32, 0, None)
    assert st == -1
    st = lg.gemm_run_config(99, 8, 8, 8, A0, 8, R, B0, 8, R, None, 8, D0, 8, F16, F32, F32, 0,
                            None)
    assert st == -8
    st = lg.gemm_run(0, 8, 8, A0, 8, R, B0, 8, R, None, 8, D0, 8, F16, F32, F32, 0, None)
    assert st == 0  # empty problem: nothing enqueued


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    monkeypatch.setattr(lg, "_lib", None)
    monkeypatch.setattr(lg, "LIB_PATH", str(tmp_path / "absent.so"))
    with pytest.raises(RuntimeError, match="not built"):
        lg.library()
