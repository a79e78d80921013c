"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (no GPU):
the CPU oracle (oracle/gemm_oracle.c, driven by tests/oracle_sanitize.c over
small and edge-case problems with exactly sized buffers) and the C ABI's
argument validation (csrc/gemm_validate.hpp, driven by
tests/validate_check.cpp with every documented status and the extreme values
where its arithmetic could overflow).  The operand-load address check runs
under the same sanitizers in test_address_cpu.py."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
TESTS = os.path.join(ROOT, "tests")
CSRC = os.path.join(ROOT, "dense_mixed_precision_tiled_amd", "csrc")
SAN = ["-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all"]


def _run(cmd, exe):
    subprocess.run(cmd, check=True)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout + r.stderr
    return r.stdout


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_sanitize")
    out = _run(["gcc", "-std=c11", "-ffp-contract=off", "-pthread"] + SAN +
               [os.path.join(ROOT, "oracle", "gemm_oracle.c"),
                os.path.join(TESTS, "oracle_sanitize.c"), "-o", exe, "-lm"], exe)
    assert "0 failures" in out, out


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_validate_under_sanitizers(tmp_path):
    exe = str(tmp_path / "validate_check")
    out = _run(["g++", "-std=c++17"] + SAN + ["-I", CSRC, os.path.join(TESTS, "validate_check.cpp"),
                                              "-o", exe], exe)
    assert "0 failures" in out, out
