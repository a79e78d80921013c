"""Summaries of rocprofv3 output for the benchmark's GEMM kernel.

Two subcommands, both reading the CSV files rocprofv3 writes with
``--output-format csv``:

``stats``   the ``--kernel-trace --stats`` kernel table, as a short Markdown
            summary (calls, mean / min / max duration per kernel) with the
            command that produced it.

``traffic`` HBM bytes per GEMM launch from two ``--pmc`` runs of
            ``bench.py --calibrate-copy`` (one with FETCH_SIZE, one with
            WRITE_SIZE; both counters are KiB per dispatch).  The same runs
            contain a plain device-to-device copy of a known size; the ratio
            of its true byte count to its counter reading calibrates the
            GEMM's counters.  The result is keyed by a hash of the HIP sources
            so that bench.py reports it only while the kernels are unchanged.

    python -m dense_mixed_precision_tiled_amd.rocprof_summary stats \\
        --csv OUT/prof/bench_kernel_stats.csv --command "..." --out profiles/x.md
    python -m dense_mixed_precision_tiled_amd.rocprof_summary traffic \\
        --fetch OUT/pmc_fetch/fetch_counter_collection.csv \\
        --write OUT/pmc_write/write_counter_collection.csv \\
        --copy-bytes 268435456 --command "..." --out profiles/traffic_gemm_4096_f16.json
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import json
import os
import statistics
import sys

PKG = os.path.dirname(os.path.abspath(__file__))


def kernel_source_hash() -> str:
    """Hash of the HIP sources (csrc/*.hip, *.hpp)."""
    csrc = os.path.join(PKG, "csrc")
    h = hashlib.sha256()
    for f in sorted(os.listdir(csrc)):
        if f.endswith((".hip", ".hpp", ".h")):
            with open(os.path.join(csrc, f), "rb") as fh:
                h.update(f.encode() + b"\0" + fh.read())
    return h.hexdigest()[:16]


def _short(name: str, width: int = 110) -> str:
    return name if len(name) <= width else name[: width - 3] + "..."


def stats(args) -> int:
    rows = list(csv.DictReader(open(args.csv)))
    lines = ["# rocprofv3 kernel statistics", "",
             "Command (run from the repository root on one MI355X):", "",
             "    " + args.command, "",
             "| kernel | calls | mean us | min us | max us | share % |",
             "|---|---|---|---|---|---|"]
    for r in rows:
        lines.append("| `%s` | %s | %.2f | %.2f | %.2f | %.1f |" % (
            _short(r["Name"]), r["Calls"], float(r["AverageNs"]) / 1e3,
            float(r["MinNs"]) / 1e3, float(r["MaxNs"]) / 1e3, float(r["Percentage"])))
    with open(args.out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))
    return 0


def _per_dispatch(path: str, counter: str):
    """{dispatch id: (kernel name, value summed over instances)}"""
    out = {}
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] != counter:
            continue
        d = out.setdefault(r["Dispatch_Id"], [r["Kernel_Name"], 0.0])
        d[1] += float(r["Counter_Value"])
    return out


def _calibrated(path: str, counter: str, kernel_substr: str, copy_substr: str,
                copy_bytes: int):
    d = _per_dispatch(path, counter)
    gemm = [v for n, v in d.values() if kernel_substr in n]
    copy = [(n, v) for n, v in d.values() if copy_substr in n.lower()]
    if not gemm or not copy:
        raise SystemExit("%s: need both GEMM (%d) and copy (%d) dispatches" %
                         (path, len(gemm), len(copy)))
    copy_kib = statistics.median(v for _, v in copy)
    factor = copy_bytes / (copy_kib * 1024.0)
    gemm_kib = statistics.median(gemm)
    return {"counter_kib": gemm_kib, "factor": factor, "bytes": gemm_kib * 1024.0 * factor,
            "copy_kernel": copy[0][0], "copy_counter_kib": copy_kib, "dispatches": len(gemm)}


def traffic(args) -> int:
    rd = _calibrated(args.fetch, "FETCH_SIZE", args.kernel, args.copy_kernel, args.copy_bytes)
    wr = _calibrated(args.write, "WRITE_SIZE", args.kernel, args.copy_kernel, args.copy_bytes)
    out = {
        "kernel_source_hash": kernel_source_hash(),
        "bytes_per_launch": rd["bytes"] + wr["bytes"],
        "read_bytes": rd["bytes"], "write_bytes": wr["bytes"],
        "fetch_size_kib": rd["counter_kib"], "write_size_kib": wr["counter_kib"],
        "fetch_factor": rd["factor"], "write_factor": wr["factor"],
        "copy_kernel": rd["copy_kernel"], "copy_bytes": args.copy_bytes,
        "command": args.command,
    }
    with open(args.out, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    print(json.dumps(out, indent=1))
    return 0


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    sub = ap.add_subparsers(dest="cmd", required=True)
    s = sub.add_parser("stats")
    s.add_argument("--csv", required=True)
    s.add_argument("--command", required=True)
    s.add_argument("--out", required=True)
    t = sub.add_parser("traffic")
    t.add_argument("--fetch", required=True)
    t.add_argument("--write", required=True)
    t.add_argument("--copy-bytes", type=int, required=True)
    t.add_argument("--kernel", default="gemm_mfma_kernel")
    t.add_argument("--copy-kernel", default="copy")
    t.add_argument("--command", required=True)
    t.add_argument("--out", required=True)
    args = ap.parse_args(argv)
    return stats(args) if args.cmd == "stats" else traffic(args)


if __name__ == "__main__":
    sys.exit(main())
