"""The operand loads' address arithmetic, checked on the host: the kernels'
loaders compose their byte offsets from the functions of
``csrc/gemm_address.hpp``; ``address_check.cpp`` composes them the same way
for every tile, thread, chunk and K-tile of a set of problems (the HGEMM
workload's ragged K among them) and checks that every 16-byte chunk read lies
inside the operand and holds one of its elements.  The LDS-DMA loads are
checked the same way on the global side (16-bit and 8-bit, both storage
orders, plain and clamped K), and simulated on the LDS side: placement,
swizzles, the transposed reads with the lane exchange probed on the GPU,
every lane's MFMA operand and, for the 8-bit transposed reads, the banks
each half-wave touches.  It also walks the
workgroup-to-tile raster (``raster_tile``) over grids, group heights, XCD
counts and the skewed column order, and checks that every tile is computed
exactly once.  Built with g++ under
AddressSanitizer and UndefinedBehaviorSanitizer."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "dense_mixed_precision_tiled_amd", "csrc")
SRC = os.path.join(ROOT, "tests", "address_check.cpp")


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_every_chunk_read_lies_inside_the_operand(tmp_path):
    exe = str(tmp_path / "address_check")
    subprocess.run(["g++", "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=all", "-I", CSRC, SRC, "-o", exe], check=True)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "0 failures" in r.stdout, r.stdout
