"""CPU tests of bench.py's contract that need no GPU: the one-GPU guard and
the compulsory-byte count behind the roofline figures."""
from __future__ import annotations

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from dense_mixed_precision_tiled_amd import workloads as W  # noqa: E402


@pytest.mark.parametrize("argv,env", [(["--gpus", "2"], {}), (["--gpus", "8"], {}),
                                      ([], {"WORLD_SIZE": "2"})])
def test_more_than_one_gpu_exits_with_a_message(argv, env):
    e = dict(os.environ, **env)
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")] + argv, env=e,
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_compulsory_bytes_of_the_headline():
    # A and B fp16 4096^2 (32 MiB each), no C, D fp32 4096^2 (64 MiB)
    prob = W.w_4096_f16("int")
    assert bench.algorithmic_bytes(prob) == 2 * 4096 * 4096 * 2 + 4096 * 4096 * 4 == 134217728


def test_compulsory_bytes_count_c_bias_and_16_bit_outputs():
    # in-place fp32 C: read once and written once
    prob = W.w_4096_bf16_inplace("int")
    assert bench.algorithmic_bytes(prob) == 2 * (2 * 4096 * 4096) + 2 * (4 * 4096 * 4096)
    # HGEMM: fp16 C and D over M x N (not the padded ld), A and B over the logical sizes
    M, N, K = 3999, 4001, 4104
    prob = W.w_hgemm(0, "int")
    assert bench.algorithmic_bytes(prob) == 2 * M * K + 2 * K * N + 2 * M * N + 2 * M * N
    # the extended epilogue's bias adds 4 bytes per column
    ep = W.make_epilogue_problem(64, 96, 32, values="int", c_values=None, bias_values="int",
                                 act=2, seed=1)
    assert bench.algorithmic_bytes(ep) == 2 * 64 * 32 + 2 * 32 * 96 + 4 * 96 + 4 * 64 * 96


def test_compulsory_bytes_of_8_bit_inputs():
    # int8 A, B (1 byte each), int32 D (4 bytes); fp8 A, B (1 byte), fp32 D
    prob = W.make_int8_problem(300, 200, 100, values="small", c_values="int", seed=2)
    assert bench.algorithmic_bytes(prob) == 300 * 100 + 100 * 200 + 2 * 4 * 300 * 200
    prob = W.make_problem(300, 200, 100, layoutB=W.COL_MAJOR, in_dtype=W.FP8_E4M3,
                          values="uniform", seed=3)
    assert bench.algorithmic_bytes(prob) == 300 * 100 + 100 * 200 + 4 * 300 * 200


def test_every_workload_has_a_description_and_bound():
    for name, (gen, desc, bound) in bench.WORKLOADS.items():
        assert desc and bound in ("mfma", "hbm", "mfma_i8", "mfma_fp8"), name
        if gen is not None:
            assert callable(getattr(W, gen)), name


@pytest.mark.parametrize("kind", ["f16_fp32", "f16_out", "i8", "fp8", "epilogue_colD", "inplace"])
def test_cpu_baseline_runs_the_matching_oracle(kind):
    """cpu_baseline times the oracle call that matches the workload's types and
    epilogue (small shapes here)."""
    if kind == "f16_fp32":
        prob = W.make_problem(48, 40, 64, values="uniform", seed=11)
    elif kind == "f16_out":
        prob = W.make_problem(48, 40, 64, acc_dtype=W.F16, out_dtype=W.F16, values="uniform",
                              c_values="normal", ldd=44, ldc=44, seed=12)
    elif kind == "i8":
        prob = W.make_int8_problem(48, 40, 64, values="full", c_values="int", seed=13)
    elif kind == "fp8":
        prob = W.make_problem(48, 40, 64, layoutB=W.COL_MAJOR, in_dtype=W.FP8_E4M3,
                              values="uniform", seed=14)
    elif kind == "epilogue_colD":
        prob = W.make_epilogue_problem(48, 40, 64, layoutD=W.COL_MAJOR, values="uniform",
                                       c_values="normal", bias_values="normal", act=2, seed=15)
    else:
        prob = W.make_problem(48, 40, 64, in_dtype=W.BF16, values="normal", c_values="normal",
                              inplace=True, seed=16)
    r = bench.cpu_baseline(prob, 0.02)
    assert r["value"] > 0 and r["kind"] == "oracle" and r["cores"] >= 1
    assert r["unit"] == ("TOP/s" if kind == "i8" else "TFLOP/s")
