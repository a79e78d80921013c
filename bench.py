#!/usr/bin/env python3
"""Benchmark of the hot path: D = A x B + C through libgemm on one MI355X.

Default workload: M = N = K = 4096, A and B fp16 row-major (lda = K,
ldb = N), uniform[-1,1] (seeded), fp32 accumulate and fp32 D, C = 0.  One
step = one gemm_run over that batch, inputs resident in HBM before the timed
region starts.  Prints ONE JSON line:

  value       = 2*M*N*K / (wall time per step) in TFLOP/s, over K steps
                launched back to back
  roofline    = the GEMM kernel's own rate: 2*M*N*K / (mean launch duration,
                HIP events around each of K further launches on the launch
                stream) against the 2.5 PFLOP/s dense fp16 MFMA peak
  cpu_baseline= the CPU oracle on a bounded sample of the same workload (the
                first rows of D), on this host's cores

    python bench.py [--gpus 1] [--steps 50] [--warmup 10] [--no-cpu-baseline]

The ceilings the GEMM is read against are workloads too (lib/libgemm_measure.so):
``--workload mfma_peak_32`` / ``mfma_peak_16`` (a stream of independent
v_mfma_f32_32x32x16_f16 / 16x16x32_f16 on random fp16 operands in registers,
one workgroup of four waves per CU) and ``--workload copy`` (a 16-byte
load/store copy of 512 MiB); ``--workload vendor_4096_f16`` times the
platform's BLAS (torch.mm with fp32 output) on the headline problem, for
context only.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "GEMM TFLOP/s (2MNK/t) and % of MI355X fp16 MFMA peak, 4096³ fp16→fp32"
PEAK_TFLOPS = 2500.0  # MI355X dense fp16/bf16 MFMA, published
COPY_BYTES = 256 << 20  # size of the calibration copy


def traffic_file(workload: str) -> str:
    return os.path.join(ROOT, "profiles", "traffic_%s.json" % workload)


def load_traffic(workload: str):
    """HBM bytes per launch from the committed counter summary of this
    workload, while the kernel sources are the ones it was taken from."""
    try:
        with open(traffic_file(workload)) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    from dense_mixed_precision_tiled_amd.rocprof_summary import kernel_source_hash
    if t.get("kernel_source_hash") != kernel_source_hash():
        return None
    return t.get("bytes_per_launch")


def cpu_baseline(prob, target_s: float):
    """Time the oracle on the first R rows of D (all N columns, full K): the
    same computation as the workload (int8 through the integer oracle, the
    extended epilogue through gemm_ex), into a host buffer of D's type."""
    import numpy as np
    import oracle

    oracle.build(force=False)
    threads = oracle.default_threads()   # every core this process may run on
    C = prob.D if prob.inplace else prob.C     # prob.D still holds the original C
    layoutD = getattr(prob, "layoutD", 0)
    dt = {W_F32: np.float32, W_I32: np.int32}.get(prob.out_dtype, np.uint16)

    def run_rows(R):
        # A and B whole: with M = R the oracle reads rows < R of A in either layout
        D = np.empty((R, prob.ldd) if layoutD == 0 else (prob.N, prob.ldd), dtype=dt)
        args = (R, prob.N, prob.K, prob.A.ravel(), prob.lda, prob.layoutA, prob.B.ravel(),
                prob.ldb, prob.layoutB, None if C is None else C.ravel(), prob.ldc)
        t0 = time.perf_counter()
        if prob.in_dtype == W_I8:
            oracle.gemm_i8(*args, getattr(prob, "layoutC", 0), D.ravel(), prob.ldd, layoutD,
                           prob.satf, nthreads=threads)
        elif getattr(prob, "act", None) is not None:
            oracle.gemm_ex(*args, prob.layoutC, D.ravel(), prob.ldd, layoutD, prob.in_dtype,
                           prob.acc_dtype, prob.out_dtype, prob.satf, prob.alpha, prob.beta,
                           prob.bias, prob.act, nthreads=threads)
        else:
            oracle.gemm(*args, D.ravel(), prob.ldd, prob.in_dtype, prob.acc_dtype,
                        prob.out_dtype, prob.satf, nthreads=threads)
        return time.perf_counter() - t0

    probe_rows = threads
    t_probe = run_rows(probe_rows)
    rows = int(max(threads, min(prob.M, probe_rows * target_s / max(t_probe, 1e-6))))
    rows = max(threads, (rows // threads) * threads)
    t = run_rows(rows)
    flops = 2.0 * rows * prob.N * prob.K
    return {
        "value": flops / t / 1e12,
        "unit": "TOP/s" if prob.in_dtype == W_I8 else "TFLOP/s",
        "cores": threads,
        "kind": "oracle",
        "sample": "first %d of %d rows of D (%d x %d outputs, K=%d), %s, %.1f s"
                  % (rows, prob.M, rows, prob.N, prob.K,
                     "exact int64 sums" if prob.in_dtype == W_I8 else "fp64 accumulate", t),
    }


# name -> (generator, description, roofline bound)
WORKLOADS = {
    "4096_f16": ("w_4096_f16", "M=N=K=4096 GEMM, fp16 row-major A and B (uniform[-1,1], "
                 "seeded), fp32 accumulate, fp32 D, C=0", "mfma"),
    "256_f16": ("w_256", "M=N=K=256 GEMM, fp16 row-major A and B (uniform[-1,1]), fp32 D, C=0",
                "mfma"),
    "4096_bf16_inplace": ("w_4096_bf16_inplace", "M=N=K=4096 GEMM, bf16 row-major A, bf16 "
                          "col-major B (normal), fp32 C updated in place", "mfma"),
    "hgemm_satf0": ("w_hgemm", "HGEMM 3999x4001x4104, fp16 accumulate/out, padded ld, 1% of "
                    "A rows x2048, satf=0", "mfma"),
    "hgemm_satf1": ("w_hgemm", "HGEMM 3999x4001x4104, fp16 accumulate/out, padded ld, 1% of "
                    "A rows x2048, satf=1", "mfma"),
    "wide": ("w_wide", "M=N=16384, K=1024 GEMM, fp16 row-major in, fp32 D", "mfma"),
    "skinny": ("w_skinny", "M=16, N=K=16384 GEMM, fp16 row-major in, fp32 D", "hbm"),
    # extended epilogue (gemm_run_ex) on the headline shape
    "4096_f16_bias_gelu": (None, "M=N=K=4096 GEMM, fp16 row-major A and B (uniform[-1,1]), "
                           "fp32 D = GELU(A x B + bias), bias N(0,1) fp32 per column", "mfma"),
    "4096_f16_colD": (None, "M=N=K=4096 GEMM, fp16 row-major A and B (uniform[-1,1]), "
                      "fp32 D column-major, C=0", "mfma"),
    # int8 x int8 -> int32
    "4096_i8": (None, "M=N=K=4096 GEMM, int8 A row-major and B column-major (uniform over "
                "[-128,127]), int32 accumulate and D, C=0", "mfma_i8"),
    # OCP fp8 E4M3 inputs, fp32 accumulate
    "4096_fp8": (None, "M=N=K=4096 GEMM, fp8 E4M3 A row-major and B column-major "
                 "(uniform[-1,1] rounded to E4M3), fp32 accumulate and D, C=0", "mfma_fp8"),
    # the same with row-major B (N-contiguous, transposed on the way to LDS)
    "4096_i8_rowB": (None, "M=N=K=4096 GEMM, int8 A and B row-major (uniform over "
                     "[-128,127]), int32 accumulate and D, C=0", "mfma_i8"),
    "4096_fp8_rowB": (None, "M=N=K=4096 GEMM, fp8 E4M3 A and B row-major (uniform[-1,1] "
                      "rounded to E4M3), fp32 accumulate and D, C=0", "mfma_fp8"),
}
# the measured ceilings (libgemm_measure): name -> (description, unit)
MEASURE_WORKLOADS = {
    "mfma_peak_32": ("MFMA stream: independent v_mfma_f32_32x32x16_f16 on random fp16 operands "
                     "held in registers, 8 waves (two per SIMD) per CU, no memory traffic",
                     "TFLOP/s"),
    "mfma_peak_16": ("MFMA stream: independent v_mfma_f32_16x16x32_f16 on random fp16 operands "
                     "held in registers, 8 waves (two per SIMD) per CU, no memory traffic",
                     "TFLOP/s"),
    "copy": ("device copy of 512 MiB with 16-byte loads and stores (read + write bytes)", "GB/s"),
    "vendor_4096_f16": ("the platform's BLAS on the headline problem, for context: torch.mm "
                        "(hipBLASLt) of the same fp16 row-major A and B with fp32 output",
                        "TFLOP/s"),
}
MEASURE_LIB = os.path.join(ROOT, "dense_mixed_precision_tiled_amd", "lib", "libgemm_measure.so")
PEAK_I8_TOPS = 5000.0  # MI355X dense int8 MFMA, published
PEAK_FP8_TFLOPS = 5000.0  # MI355X dense fp8 MFMA, published
PEAK_HBM_GBS = 8000.0  # MI355X HBM3E, published
W_F32, W_I8, W_I32, W_FP8_E4M3, W_FP8_E5M2 = 0, 3, 4, 5, 6  # gemm_dtype_t codes


def make_workload(W, name):
    gen, desc, bound = WORKLOADS[name]
    if name == "4096_f16_bias_gelu":
        prob = W.make_epilogue_problem(4096, 4096, 4096, values="uniform", c_values=None,
                                       bias_values="normal", act=2, ldd=4096, seed=20330)
    elif name == "4096_fp8":
        prob = W.make_problem(4096, 4096, 4096, layoutA=0, layoutB=1, in_dtype=W.FP8_E4M3,
                              values="uniform", seed=20360)
    elif name == "4096_i8":
        prob = W.make_int8_problem(4096, 4096, 4096, values="full", c_values=None, seed=20350)
    elif name == "4096_i8_rowB":
        prob = W.make_int8_problem(4096, 4096, 4096, layoutB=0, values="full", c_values=None,
                                   seed=20370)
    elif name == "4096_fp8_rowB":
        prob = W.make_problem(4096, 4096, 4096, layoutA=0, layoutB=0, in_dtype=W.FP8_E4M3,
                              values="uniform", seed=20380)
    elif name == "4096_f16_colD":
        prob = W.make_epilogue_problem(4096, 4096, 4096, layoutD=1, values="uniform",
                                       c_values=None, bias_values=None, ldd=4096, seed=20340)
    elif name.startswith("hgemm"):
        prob = getattr(W, gen)(int(name[-1]), "uniform")
    elif name == "4096_bf16_inplace":
        prob = getattr(W, gen)("normal")
    else:
        prob = getattr(W, gen)("uniform")
    return prob, desc, bound


def algorithmic_bytes(prob) -> int:
    """Compulsory HBM bytes: A and B once, C read once (if any), the bias once
    (if any), D written once, each at its element size (1 byte for int8 and
    fp8 inputs, 2 for fp16/bf16; 4 for fp32 and int32 C/D, 2 for fp16/bf16)."""
    isz = 1 if prob.in_dtype in (W_I8, W_FP8_E4M3, W_FP8_E5M2) else 2
    osz = 4 if prob.out_dtype in (W_F32, W_I32) else 2
    c = prob.M * prob.N * osz if prob.C is not None else 0
    bias = 4 * prob.N if getattr(prob, "bias", None) is not None else 0
    return isz * (prob.M * prob.K + prob.K * prob.N) + c + bias + prob.M * prob.N * osz


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run a plain 256 MiB device-to-device copy (counter calibration)")
    ap.add_argument("--autotune", action="store_true",
                    help="run gemm_autotune on the workload first (untimed) and time the "
                         "entry it records")
    ap.add_argument("--config", default=None,
                    help="force this tile-table entry (by name) instead of the dispatcher's "
                         "choice, for comparisons between entries")
    ap.add_argument("--workload", default="4096_f16",
                    choices=sorted(WORKLOADS) + sorted(MEASURE_WORKLOADS),
                    help="workload to time (default: the headline 4096^3 fp16->fp32)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: libgemm has no multi-GPU path "
              "(the GEMM shards by output tiles with no collective; see the design notes). "
              "Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import dense_mixed_precision_tiled_amd as lg
    from dense_mixed_precision_tiled_amd import workloads as W

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    lg.library()
    if args.workload in MEASURE_WORKLOADS:
        measure(args)
        return

    prob, desc, bound = make_workload(W, args.workload)
    dev = torch.device("cuda:0")
    def to_dev(x):  # 16-bit patterns travel as int16; everything else as is
        return torch.from_numpy(x.view(np.int16) if x.dtype == np.uint16 else x).to(dev)

    A, B, D = to_dev(prob.A), to_dev(prob.B), to_dev(prob.D)
    if prob.inplace:
        C = D
    elif prob.C is not None:
        C = to_dev(prob.C)
    else:
        C = None
    stream = torch.cuda.current_stream()
    epi = getattr(prob, "act", None) is not None  # an extended-epilogue workload
    if epi:
        bias = None if prob.bias is None else torch.from_numpy(prob.bias).to(dev)
        epilogue = lg.GemmEpilogue(prob.alpha, prob.beta, 0 if bias is None else bias.data_ptr(),
                                   prob.act, prob.layoutC, prob.layoutD)
        call = (prob.M, prob.N, prob.K, A.data_ptr(), prob.lda, prob.layoutA, B.data_ptr(),
                prob.ldb, prob.layoutB, None if C is None else C.data_ptr(), prob.ldc,
                D.data_ptr(), prob.ldd, prob.in_dtype, prob.acc_dtype, prob.out_dtype,
                prob.satf, epilogue, stream.cuda_stream)
        run = lg.gemm_run_ex
    else:
        call = (prob.M, prob.N, prob.K, A.data_ptr(), prob.lda, prob.layoutA, B.data_ptr(),
                prob.ldb, prob.layoutB, None if C is None else C.data_ptr(), prob.ldc,
                D.data_ptr(), prob.ldd, prob.in_dtype, prob.acc_dtype, prob.out_dtype,
                prob.satf, stream.cuda_stream)
        run = lg.gemm_run
    cfg = lg.gemm_select_config(prob.M, prob.N, prob.K, prob.layoutA, prob.layoutB,
                                prob.in_dtype, prob.acc_dtype, prob.out_dtype)
    if args.config is not None:
        names = [lg.gemm_config_name(i) for i in range(lg.gemm_num_configs())]
        if args.config not in names:
            raise SystemExit("unknown --config %r; entries: %s" % (args.config, ", ".join(names)))
        cfg = names.index(args.config)
        forced = cfg
        run = ((lambda *a: lg.gemm_run_ex_config(forced, *a)) if epi
               else (lambda *a: lg.gemm_run_config(forced, *a)))

    tuned = None
    if args.autotune:
        ex_call = call if epi else call[:-1] + (None, call[-1])
        t0 = time.perf_counter()
        st, tuned = lg.gemm_autotune(*ex_call[:-1], 5, ex_call[-1])
        tune_s = time.perf_counter() - t0
        if st != 0:
            raise lg.GemmError(st, "gemm_autotune")
        cfg = tuned

    if args.calibrate_copy:
        src = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    for _ in range(args.warmup):
        st = run(*call)
        if st != 0:
            raise lg.GemmError(st)
    torch.cuda.synchronize()

    # timed region: K steps back to back (value = whole-job throughput)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        st = run(*call)
        if st != 0:
            raise lg.GemmError(st)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    # the kernel's own duration: K more launches, each bracketed by HIP events
    # on the launch stream (events between launches would stretch the timed
    # region above, so they get a pass of their own)
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    for i in range(args.steps):
        starts[i].record(stream)
        st = run(*call)
        ends[i].record(stream)
        if st != 0:
            raise lg.GemmError(st)
    torch.cuda.synchronize()

    durations_ms = [s.elapsed_time(e) for s, e in zip(starts, ends)]
    mean_ms = sum(durations_ms) / len(durations_ms)
    ms_per_step = wall * 1e3 / args.steps
    flop = float(prob.flops)
    value = flop / (ms_per_step * 1e-3) / 1e12
    achieved = flop / (mean_ms * 1e-3) / 1e12
    traffic = load_traffic(args.workload)
    nbytes = algorithmic_bytes(prob)
    if bound == "mfma_fp8":
        roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_FP8_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / PEAK_FP8_TFLOPS, 4)}
    elif bound == "mfma_i8":
        roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_I8_TOPS,
                "unit": "TOP/s", "frac": round(achieved / PEAK_I8_TOPS, 4)}
    elif bound == "hbm":
        roof = {"bound": "hbm", "achieved": round(nbytes / (mean_ms * 1e-3) / 1e9, 1),
                "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(nbytes / (mean_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}
    else:
        roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / PEAK_TFLOPS, 4)}

    out = {
        "metric": METRIC if args.workload == "4096_f16" else
        "GEMM %s (2MNK/t), workload %s" % ("TOP/s" if prob.in_dtype == 3 else "TFLOP/s",
                                           args.workload),
        "value": round(value, 2),
        "unit": "TOP/s" if prob.in_dtype == 3 else "TFLOP/s",
        "pct_of_peak": round(100.0 * value / (PEAK_I8_TOPS if prob.in_dtype == 3 else
                                               PEAK_FP8_TFLOPS if prob.in_dtype in (5, 6)
                                               else PEAK_TFLOPS), 2),
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {2: "bf16", 3: "i8", 5: "fp8_e4m3", 6: "fp8_e5m2"}.get(prob.in_dtype, "f16"),
        "data": "synthetic",
        "config": {
            "workload": desc,
            "M": prob.M, "N": prob.N, "K": prob.K,
            "tile_config": lg.gemm_config_name(cfg),
            "autotuned": None if tuned is None else {"entry": lg.gemm_config_name(tuned),
                                                     "tuning_s": round(tune_s, 3)},
        },
        "roofline": dict(roof, **{
            "traffic": traffic,
            "algorithmic_bytes": nbytes,
            "kernel": "libgemm entry %s" % lg.gemm_config_name(cfg),
            "launch_ms_mean": round(mean_ms, 5),
            "launch_ms_min": round(min(durations_ms), 5),
            "launch_ms_median": round(sorted(durations_ms)[len(durations_ms) // 2], 5),
        }),
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline and args.workload == "4096_f16":
        out["cpu_baseline"] = cpu_baseline(prob, args.cpu_seconds)
    print(json.dumps(out), flush=True)


def measure(args):
    """Time a ceiling workload of libgemm_measure with the same protocol (K
    back-to-back steps for `value`, K more launches bracketed by HIP events
    for the per-launch rate)."""
    import ctypes

    import numpy as np
    import torch

    if not os.path.exists(MEASURE_LIB):
        raise RuntimeError("libgemm_measure.so is not built; run "
                           "`python -m dense_mixed_precision_tiled_amd.build`")
    lib = ctypes.CDLL(MEASURE_LIB)
    vp, i64 = ctypes.c_void_p, ctypes.c_int64
    lib.gemm_measure_mfma_stream.argtypes = [ctypes.c_int] * 4 + [vp, vp, vp]
    lib.gemm_measure_mfma_flops.restype = i64
    lib.gemm_measure_mfma_flops.argtypes = [ctypes.c_int] * 4
    lib.gemm_measure_copy.argtypes = [vp, vp, i64, vp]
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    desc, unit = MEASURE_WORKLOADS[args.workload]
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    if args.workload.startswith("mfma_peak"):
        mf = int(args.workload.rsplit("_", 1)[1])
        rng = np.random.default_rng(20260)
        ops = (rng.random(32768, dtype=np.float32) * 2 - 1).astype(np.float16)   # 64 KiB
        operands = torch.from_numpy(ops.view(np.int16)).to(dev)
        blocks, threads, iters = cus, 512, 10000
        out = torch.empty(blocks * threads, dtype=torch.float32, device=dev)
        work = float(lib.gemm_measure_mfma_flops(mf, blocks, threads, iters))

        def launch():
            return lib.gemm_measure_mfma_stream(mf, blocks, threads, iters, operands.data_ptr(),
                                                out.data_ptr(), stream.cuda_stream)
        peak, bound, dtype = PEAK_TFLOPS, "mfma", "f16"
        config = {"workload": desc, "mfma": "32x32x16" if mf == 32 else "16x16x32",
                  "workgroups": blocks, "threads": threads, "rounds": iters}
    elif args.workload == "vendor_4096_f16":
        from dense_mixed_precision_tiled_amd import workloads as W
        prob = W.w_4096_f16("uniform")
        A = torch.from_numpy(prob.A.view(np.int16)).to(dev).view(torch.float16)
        B = torch.from_numpy(prob.B.view(np.int16)).to(dev).view(torch.float16)
        D = torch.empty(prob.M, prob.N, dtype=torch.float32, device=dev)
        work = float(prob.flops)

        def launch():
            torch.mm(A, B, out_dtype=torch.float32, out=D)
            return 0
        peak, bound, dtype = PEAK_TFLOPS, "mfma", "f16"
        config = {"workload": desc, "M": prob.M, "N": prob.N, "K": prob.K}
    else:
        nbytes = 512 << 20
        src = torch.empty(nbytes // 4, dtype=torch.float32, device=dev).uniform_()
        dst = torch.empty_like(src)
        work = 2.0 * nbytes

        def launch():
            return lib.gemm_measure_copy(src.data_ptr(), dst.data_ptr(), nbytes,
                                         stream.cuda_stream)
        peak, bound, dtype = PEAK_HBM_GBS, "hbm", "u8"
        config = {"workload": desc, "bytes_copied": nbytes}
    scale = 1e12 if unit == "TFLOP/s" else 1e9
    for _ in range(args.warmup):
        if launch() != 0:
            raise RuntimeError("measurement launch failed")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        if launch() != 0:
            raise RuntimeError("measurement launch failed")
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    for i in range(args.steps):
        starts[i].record(stream)
        launch()
        ends[i].record(stream)
    torch.cuda.synchronize()
    durations_ms = [a.elapsed_time(b) for a, b in zip(starts, ends)]
    mean_ms = sum(durations_ms) / len(durations_ms)
    achieved = work / (mean_ms * 1e-3) / scale
    out = {
        "metric": ("vendor library TFLOP/s (2MNK/t), workload %s" % args.workload
                   if args.workload.startswith("vendor") else
                   "%s ceiling, workload %s" % ("MFMA" if bound == "mfma" else "HBM copy",
                                                args.workload)),
        "value": round(work * args.steps / wall / scale, 2), "unit": unit, "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3 / args.steps, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": dtype, "data": "synthetic",
        "config": config,
        "roofline": {"bound": bound, "achieved": round(achieved, 2), "peak": peak, "unit": unit,
                     "frac": round(achieved / peak, 4), "traffic": None,
                     "launch_ms_mean": round(mean_ms, 5),
                     "launch_ms_min": round(min(durations_ms), 5)},
        "cpu_baseline": None,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
