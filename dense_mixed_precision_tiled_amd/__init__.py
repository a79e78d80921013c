"""Python binding of libgemm (tiled mixed-precision D = A x B + C on MI355X).

Argument marshalling only: every step of the multiply-accumulate runs in the
HIP kernels of ``lib/libgemm.so``.  The functions keep the C names and
argument order of ``include/libgemm.h``; pointers are passed as integers
(device addresses, e.g. ``tensor.data_ptr()``) and the stream as the integer
value of a ``hipStream_t`` (``torch.cuda.current_stream().cuda_stream``).

The library is loaded on first use.  When it is missing this raises: there
is no fallback path.
"""
from __future__ import annotations

import ctypes
import os

# PyTorch-ROCm ships its own HIP runtime with the same soname as /opt/rocm's;
# importing torch first makes libgemm bind to that one runtime, so torch's
# streams and allocations are valid handles for libgemm.
import torch  # noqa: F401

__all__ = [
    "GEMM_ROW_MAJOR", "GEMM_COL_MAJOR", "GEMM_F32", "GEMM_F16", "GEMM_BF16", "GEMM_I8",
    "GEMM_I32", "GEMM_FP8_E4M3", "GEMM_FP8_E5M2",
    "GEMM_OK", "GemmError", "LIB_PATH", "library",
    "gemm_run", "gemm_run_noalloc", "gemm_run_config", "gemm_validate", "gemm_status_string",
    "gemm_num_configs", "gemm_config_name", "gemm_select_config",
    "GEMM_ACT_NONE", "GEMM_ACT_RELU", "GEMM_ACT_GELU", "GemmEpilogue",
    "gemm_run_ex", "gemm_run_ex_config", "gemm_validate_ex",
    "gemm_autotune", "gemm_autotune_lookup", "gemm_autotune_clear",
]

GEMM_ROW_MAJOR, GEMM_COL_MAJOR = 0, 1
GEMM_F32, GEMM_F16, GEMM_BF16, GEMM_I8, GEMM_I32 = 0, 1, 2, 3, 4
GEMM_FP8_E4M3, GEMM_FP8_E5M2 = 5, 6
GEMM_OK = 0
GEMM_ACT_NONE, GEMM_ACT_RELU, GEMM_ACT_GELU = 0, 1, 2
STATUS_NAMES = {
    0: "GEMM_OK", -1: "GEMM_ERR_INVALID_DIM", -2: "GEMM_ERR_INVALID_LD",
    -3: "GEMM_ERR_NULL_PTR", -4: "GEMM_ERR_UNSUPPORTED", -5: "GEMM_ERR_INVALID_LAYOUT",
    -6: "GEMM_ERR_ALIASING", -7: "GEMM_ERR_HIP", -8: "GEMM_ERR_INVALID_CONFIG",
    -9: "GEMM_ERR_SCRATCH_TOO_SMALL",
}

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "lib", "libgemm.so")


class GemmEpilogue(ctypes.Structure):
    """gemm_epilogue_t: D = act(alpha * A x B + beta * C + bias), C/D layouts.

    ``bias`` is a device address (int) of N fp32 values, or 0 for none."""
    _fields_ = [("alpha", ctypes.c_float), ("beta", ctypes.c_float),
                ("bias", ctypes.c_void_p), ("activation", ctypes.c_int),
                ("layoutC", ctypes.c_int), ("layoutD", ctypes.c_int)]

    def __init__(self, alpha=1.0, beta=1.0, bias=0, activation=GEMM_ACT_NONE,
                 layoutC=GEMM_ROW_MAJOR, layoutD=GEMM_ROW_MAJOR):
        super().__init__(alpha, beta, bias or None, activation, layoutC, layoutD)


# Exported symbols and their C signatures (mirrors include/libgemm.h).
_i64, _int, _vp, _cp = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p, ctypes.c_char_p
_GEMM_ARGS = [_i64, _i64, _i64, _vp, _i64, _int, _vp, _i64, _int, _vp, _i64, _vp, _i64,
              _int, _int, _int, _int, _vp]
SIGNATURES = {
    "gemm_run": (_int, _GEMM_ARGS),
    "gemm_run_noalloc": (_int, _GEMM_ARGS),
    "gemm_run_config": (_int, [_int] + _GEMM_ARGS),
    "gemm_validate": (_int, [_i64, _i64, _i64, _vp, _i64, _int, _vp, _i64, _int, _vp, _i64,
                             _vp, _i64, _int, _int, _int]),
    "gemm_status_string": (_cp, [_int]),
    "gemm_num_configs": (_int, []),
    "gemm_config_name": (_cp, [_int]),
    "gemm_select_config": (_int, [_i64, _i64, _i64, _int, _int, _int, _int, _int]),
    "gemm_run_ex": (_int, _GEMM_ARGS[:-1] + [ctypes.POINTER(GemmEpilogue), _vp]),
    "gemm_run_ex_config": (_int, [_int] + _GEMM_ARGS[:-1] + [ctypes.POINTER(GemmEpilogue), _vp]),
    "gemm_validate_ex": (_int, [_i64, _i64, _i64, _vp, _i64, _int, _vp, _i64, _int, _vp, _i64,
                                _vp, _i64, _int, _int, _int, ctypes.POINTER(GemmEpilogue)]),
    "gemm_autotune": (_int, _GEMM_ARGS[:-1] + [ctypes.POINTER(GemmEpilogue), _int,
                                              ctypes.POINTER(_int), _vp]),
    "gemm_autotune_lookup": (_int, [_i64, _i64, _i64, _int, _int, _int, _int, _int, _int]),
    "gemm_autotune_clear": (None, []),
}


class GemmError(RuntimeError):
    def __init__(self, status: int, where: str = "gemm_run"):
        self.status = status
        super().__init__("%s failed: %s (%s)" % (where, STATUS_NAMES.get(status, status),
                                                gemm_status_string(status)))


_lib = None


def library() -> ctypes.CDLL:
    """Load lib/libgemm.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                "libgemm.so is not built (%s); run "
                "`python -m dense_mixed_precision_tiled_amd.build`" % LIB_PATH)
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def gemm_run(M, N, K, A, lda, layoutA, B, ldb, layoutB, C, ldc, D, ldd,
             in_dtype, acc_dtype, out_dtype, satf, stream) -> int:
    """Enqueue D = A x B + C; returns the gemm_status_t code."""
    return library().gemm_run(M, N, K, A, lda, layoutA, B, ldb, layoutB, C or None, ldc,
                              D, ldd, in_dtype, acc_dtype, out_dtype, int(satf), stream or None)


def gemm_run_noalloc(M, N, K, A, lda, layoutA, B, ldb, layoutB, C, ldc, D, ldd,
                     in_dtype, acc_dtype, out_dtype, satf, stream) -> int:
    """gemm_run with no device allocation (split-K partial sums in the
    library's fixed 32 MiB scratch); returns the status code."""
    return library().gemm_run_noalloc(M, N, K, A, lda, layoutA, B, ldb, layoutB, C or None, ldc,
                                      D, ldd, in_dtype, acc_dtype, out_dtype, int(satf),
                                      stream or None)


def gemm_run_config(config_id, M, N, K, A, lda, layoutA, B, ldb, layoutB, C, ldc, D, ldd,
                    in_dtype, acc_dtype, out_dtype, satf, stream) -> int:
    """gemm_run with the tile-table entry forced; returns the status code."""
    return library().gemm_run_config(config_id, M, N, K, A, lda, layoutA, B, ldb, layoutB,
                                     C or None, ldc, D, ldd, in_dtype, acc_dtype, out_dtype,
                                     int(satf), stream or None)


def gemm_validate(M, N, K, A, lda, layoutA, B, ldb, layoutB, C, ldc, D, ldd,
                  in_dtype, acc_dtype, out_dtype) -> int:
    """Host-only argument check (no device needed); returns the status code."""
    return library().gemm_validate(M, N, K, A or None, lda, layoutA, B or None, ldb, layoutB,
                                   C or None, ldc, D or None, ldd, in_dtype, acc_dtype,
                                   out_dtype)


def gemm_status_string(status: int) -> str:
    return library().gemm_status_string(status).decode()


def gemm_num_configs() -> int:
    return library().gemm_num_configs()


def gemm_config_name(config_id: int):
    s = library().gemm_config_name(config_id)
    return None if s is None else s.decode()


def gemm_select_config(M, N, K, layoutA, layoutB, in_dtype, acc_dtype, out_dtype) -> int:
    return library().gemm_select_config(M, N, K, layoutA, layoutB, in_dtype, acc_dtype,
                                        out_dtype)


def _epi_ref(epi):
    return None if epi is None else ctypes.byref(epi)


def gemm_run_ex(M, N, K, A, lda, layoutA, B, ldb, layoutB, C, ldc, D, ldd,
                in_dtype, acc_dtype, out_dtype, satf, epi, stream) -> int:
    """Enqueue D = act(alpha * A x B + beta * C + bias) (``epi``: a GemmEpilogue
    or None for the plain gemm_run); returns the status code."""
    return library().gemm_run_ex(M, N, K, A, lda, layoutA, B, ldb, layoutB, C or None, ldc,
                                 D, ldd, in_dtype, acc_dtype, out_dtype, int(satf),
                                 _epi_ref(epi), stream or None)


def gemm_run_ex_config(config_id, M, N, K, A, lda, layoutA, B, ldb, layoutB, C, ldc, D, ldd,
                       in_dtype, acc_dtype, out_dtype, satf, epi, stream) -> int:
    """gemm_run_ex with the tile-table entry forced; returns the status code."""
    return library().gemm_run_ex_config(config_id, M, N, K, A, lda, layoutA, B, ldb, layoutB,
                                        C or None, ldc, D, ldd, in_dtype, acc_dtype, out_dtype,
                                        int(satf), _epi_ref(epi), stream or None)


def gemm_validate_ex(M, N, K, A, lda, layoutA, B, ldb, layoutB, C, ldc, D, ldd,
                     in_dtype, acc_dtype, out_dtype, epi) -> int:
    """Host-only argument check of gemm_run_ex; returns the status code."""
    return library().gemm_validate_ex(M, N, K, A or None, lda, layoutA, B or None, ldb,
                                      layoutB, C or None, ldc, D or None, ldd, in_dtype,
                                      acc_dtype, out_dtype, _epi_ref(epi))


def gemm_autotune(M, N, K, A, lda, layoutA, B, ldb, layoutB, C, ldc, D, ldd,
                  in_dtype, acc_dtype, out_dtype, satf, epi, reps, stream):
    """Time every table entry on this call, record the fastest for the
    signature; returns (status, chosen entry).  Synchronises the stream."""
    out = ctypes.c_int(-1)
    st = library().gemm_autotune(M, N, K, A, lda, layoutA, B, ldb, layoutB, C or None, ldc,
                                 D, ldd, in_dtype, acc_dtype, out_dtype, int(satf),
                                 _epi_ref(epi), int(reps), ctypes.byref(out), stream or None)
    return st, out.value


def gemm_autotune_lookup(M, N, K, layoutA, layoutB, in_dtype, acc_dtype, out_dtype,
                         layoutD=GEMM_ROW_MAJOR) -> int:
    """The recorded entry for this signature, or -1."""
    return library().gemm_autotune_lookup(M, N, K, layoutA, layoutB, in_dtype, acc_dtype,
                                          out_dtype, layoutD)


def gemm_autotune_clear() -> None:
    library().gemm_autotune_clear()
