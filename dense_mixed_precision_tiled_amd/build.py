"""Build libgemm.so for gfx950 with hipcc (cross-compiles; no GPU needed).

    python -m dense_mixed_precision_tiled_amd.build

Objects go to <repo>/_build/libgemm/, the library to
dense_mixed_precision_tiled_amd/lib/libgemm.so (in-tree, so a snapshot of the
tree carries it to the machine that runs it).  The measurement kernels
(csrc/measure/, not part of libgemm) go to lib/libgemm_measure.so.
"""
from __future__ import annotations

import concurrent.futures
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIBDIR = os.path.join(PKG, "lib")
LIB = os.path.join(LIBDIR, "libgemm.so")
MEASURE_LIB = os.path.join(LIBDIR, "libgemm_measure.so")
MEASURE_SRC = os.path.join(CSRC, "measure", "measure_kernels.hip")
OBJDIR = os.path.join(ROOT, "_build", "libgemm")

ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# -packed-fp32-ops: keep hipcc from forming v_pk_{add,mul,fma}_f32.
FLAGS = ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wall", "-Wextra", "-Wno-unused-command-line-argument"]


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def _compile(src: str) -> str:
    obj = os.path.join(OBJDIR, os.path.basename(src) + ".o")
    cmd = [HIPCC] + FLAGS + ["-I", os.path.join(ROOT, "include"), "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed on %s:\n%s\n%s" % (src, r.stdout, r.stderr))
    # pass compiler warnings on (the host pass's note about the packed-fp32
    # target feature, which it does not know, is expected)
    warn = [ln for ln in r.stderr.splitlines()
            if "warning" in ln and "packed-fp32" not in ln and "warning generated" not in ln
            and "warnings generated" not in ln]
    if warn:
        print("\n".join(warn), file=sys.stderr)
    return obj


def build(jobs: int | None = None, verbose: bool = False) -> str:
    os.makedirs(OBJDIR, exist_ok=True)
    os.makedirs(LIBDIR, exist_ok=True)
    srcs = sources()
    jobs = jobs or min(len(srcs) + 1, max(1, min(8, os.cpu_count() or 1)))
    with concurrent.futures.ThreadPoolExecutor(jobs) as ex:
        measure = ex.submit(_compile, MEASURE_SRC)
        objs = list(ex.map(_compile, srcs))
        mobj = measure.result()
    _link([mobj], MEASURE_LIB)
    _link(objs, LIB)
    if verbose:
        print("built", LIB, "and", MEASURE_LIB)
    return LIB


def _link(objs, out: str):
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s\n%s" % (r.stdout, r.stderr))
    os.replace(tmp, out)


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
