"""Summaries of rocprofv3 output for the benchmark's GEMM kernels.

Three subcommands, all reading the CSV files rocprofv3 writes with
``--output-format csv``:

``stats``    the ``--kernel-trace --stats`` kernel table, as a short Markdown
             summary (calls, mean / min / max duration per kernel) with the
             command that produced it; ``--bytes`` / ``--flop`` per launch add
             the launch's GB/s or TFLOP/s over the summed mean durations of
             the kernels one launch runs.

``traffic``  HBM bytes per GEMM launch from two ``--pmc`` runs of
             ``bench.py --calibrate-copy`` (one with FETCH_SIZE, one with
             WRITE_SIZE; both counters are KiB per dispatch).  The same runs
             contain a plain device-to-device copy of a known size; the ratio
             of its true byte count to its counter reading calibrates the
             GEMM's counters.  A launch is one dispatch of each library kernel
             (a split-K launch has two), so the per-launch figure adds the
             median dispatch of each kernel.  The result is keyed by a hash of
             the HIP sources so that bench.py reports it only while the
             kernels are unchanged.

``counters`` a Markdown table of hardware counters per kernel from any number
             of ``--pmc`` runs of one workload, with the figures derived from
             them: MFMA busy fraction and effective clock, MFMA instruction
             count against the closed form, LDS bank-conflict share, L2 hit
             rate, the share of L2 read requests that go to DRAM, and
             calibrated HBM bytes.

    python -m dense_mixed_precision_tiled_amd.rocprof_summary stats \\
        --csv OUT/prof/bench_kernel_stats.csv --command "..." --out profiles/x.md
    python -m dense_mixed_precision_tiled_amd.rocprof_summary traffic \\
        --fetch OUT/pmc_fetch/fetch_counter_collection.csv \\
        --write OUT/pmc_write/write_counter_collection.csv \\
        --copy-bytes 268435456 --command "..." --out profiles/traffic_4096_f16.json
    python -m dense_mixed_precision_tiled_amd.rocprof_summary counters \\
        --pmc OUT/p1/a_counter_collection.csv --command "..." \\
        --pmc OUT/p2/a_counter_collection.csv --command "..." \\
        --flop 137438953472 --mfma-flop 32768 --copy-bytes 268435456 \\
        --title "..." --out profiles/x_counters.md
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import json
import os
import statistics
import sys
from collections import OrderedDict

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_KERNELS = "libgemm::"  # every kernel of the GEMM library is in this namespace


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
    lines = ["# rocprofv3 kernel statistics", ""]
    if args.title:
        lines += [args.title, ""]
    lines += ["Command (run from the repository root on one MI355X):", "",
              "    " + args.command, "",
              "| kernel | calls | mean us | min us | max us | share % |",
              "|---|---|---|---|---|---|"]
    launch_ns = 0.0
    for r in rows:
        mean_ns = float(r["AverageNs"])
        if args.kernel in r["Name"]:
            launch_ns += mean_ns
        lines.append("| `%s` | %s | %.2f | %.2f | %.2f | %.1f |" % (
            _short(r["Name"]), r["Calls"], mean_ns / 1e3,
            float(r["MinNs"]) / 1e3, float(r["MaxNs"]) / 1e3, float(r["Percentage"])))
    if launch_ns and (args.bytes or args.flop):
        # one launch runs each matching kernel once (a split-K launch has two)
        rate = []
        if args.flop:
            rate.append("%.1f TFLOP/s (%d FLOP)" % (args.flop / launch_ns / 1e3, args.flop))
        if args.bytes:
            rate.append("%.1f GB/s (%d algorithmic bytes)" % (args.bytes / launch_ns, args.bytes))
        lines += ["", "Per launch (the mean durations of the kernels matching `%s` added): "
                  "%.2f us, %s." % (args.kernel, launch_ns / 1e3, ", ".join(rate))]
    with open(args.out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))
    return 0


# ---------------------------------------------------------------- counters

def _load(paths):
    """{(kernel name, counter): {dispatch id: summed value}} and
    {(kernel name, path): {dispatch id: duration ns}} over the CSV files."""
    vals = OrderedDict()
    durs = OrderedDict()
    for path in paths:
        for r in csv.DictReader(open(path)):
            key = (r["Kernel_Name"], r["Counter_Name"])
            d = (path, r["Dispatch_Id"])
            per = vals.setdefault(key, OrderedDict())
            per[d] = per.get(d, 0.0) + float(r["Counter_Value"])
            try:
                dt = float(r["End_Timestamp"]) - float(r["Start_Timestamp"])
            except (KeyError, ValueError, TypeError):
                continue
            if dt > 0:
                durs.setdefault((r["Kernel_Name"], path), OrderedDict())[d] = dt
    return vals, durs


def _median_by_counter(vals, kernel):
    return {c: statistics.median(per.values()) for (k, c), per in vals.items() if k == kernel}


def _copy_factor(vals, counter, copy_substr, copy_bytes):
    copies = [statistics.median(per.values()) for (k, c), per in vals.items()
              if c == counter and copy_substr in k.lower()]
    if not copies or copies[0] <= 0:
        return None
    return copy_bytes / (copies[0] * 1024.0)


def derived(med, args, dur_ns, fetch_factor, write_factor):
    """Rows (figure, value, how) derived from one kernel's median counters."""
    out = []
    cyc = None
    if "GRBM_GUI_ACTIVE" in med:
        cyc = med["GRBM_GUI_ACTIVE"] / args.xcds
        out.append(("GPU cycles per dispatch", "%.0f" % cyc,
                    "GRBM_GUI_ACTIVE / %d XCDs" % args.xcds))
        if dur_ns:
            out.append(("effective clock", "%.3f GHz" % (cyc / dur_ns),
                        "cycles / dispatch duration (%.2f us, same run)" % (dur_ns / 1e3)))
    busy = med.get("SQ_VALU_MFMA_BUSY_CYCLES")
    simds = args.cus * args.simds
    if busy is not None and cyc:
        out.append(("MFMA busy", "%.3f" % (busy / (simds * cyc)),
                    "SQ_VALU_MFMA_BUSY_CYCLES / (%d SIMDs x GPU cycles)" % simds))
    cu = med.get("SQ_BUSY_CU_CYCLES")
    if cu:
        per_cu = cu / args.cus
        out.append(("busy cycles per CU", "%.0f" % per_cu, "SQ_BUSY_CU_CYCLES / %d CUs" % args.cus))
        if dur_ns:
            out.append(("clock while busy", "%.3f GHz" % (per_cu / dur_ns),
                        "busy cycles per CU / dispatch duration"))
        if busy is not None:
            out.append(("MFMA busy per busy CU cycle", "%.3f" % (busy / (simds * per_cu)),
                        "SQ_VALU_MFMA_BUSY_CYCLES / (%d SIMDs x busy cycles per CU)" % simds))
    if busy is not None and args.flop:
        out.append(("FLOP per MFMA busy cycle", "%.1f" % (args.flop / busy) if busy else "-",
                    "closed-form FLOP / SQ_VALU_MFMA_BUSY_CYCLES"))
    if args.flop and args.mfma_flop:
        closed = args.flop / args.mfma_flop
        for c in sorted(med):
            if c.startswith("SQ_INSTS_VALU_MFMA_") and "MOPS" not in c and med[c] > 0:
                out.append(("MFMA instructions / closed form", "%.0f / %.0f = %.4f" % (
                    med[c], closed, med[c] / closed),
                    "%s against 2MNK / %d FLOP per instruction" % (c, args.mfma_flop)))
        for c in sorted(med):
            if c.startswith("SQ_INSTS_VALU_MFMA_MOPS_") and med[c] > 0:
                out.append(("FLOP per %s unit" % c, "%.1f" % (args.flop / med[c]),
                            "closed-form FLOP / counter"))
    if "SQ_LDS_BANK_CONFLICT" in med and med.get("SQ_LDS_IDX_ACTIVE"):
        out.append(("LDS bank-conflict share", "%.4f" % (
            med["SQ_LDS_BANK_CONFLICT"] / med["SQ_LDS_IDX_ACTIVE"]),
            "SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE (cycles)"))
    hit, miss = med.get("TCC_HIT_sum"), med.get("TCC_MISS_sum")
    if hit is not None and miss is not None and hit + miss > 0:
        out.append(("L2 hit rate", "%.3f" % (hit / (hit + miss)), "TCC_HIT / (TCC_HIT + TCC_MISS)"))
    rd, rdd = med.get("TCC_EA0_RDREQ_sum"), med.get("TCC_EA0_RDREQ_DRAM_sum")
    if rd and rdd is not None:
        out.append(("L2 read requests to DRAM", "%.3f" % (rdd / rd),
                    "TCC_EA0_RDREQ_DRAM / TCC_EA0_RDREQ"))
    wr, wrd = med.get("TCC_EA0_WRREQ_sum"), med.get("TCC_EA0_WRREQ_DRAM_sum")
    if wr and wrd is not None:
        out.append(("L2 write requests to DRAM", "%.3f" % (wrd / wr),
                    "TCC_EA0_WRREQ_DRAM / TCC_EA0_WRREQ"))
    rb = wb = None
    if "FETCH_SIZE" in med and fetch_factor:
        rb = med["FETCH_SIZE"] * 1024.0 * fetch_factor
        out.append(("HBM read bytes", "%.4g" % rb,
                    "FETCH_SIZE KiB x 1024 x copy calibration %.4f" % fetch_factor))
    if "WRITE_SIZE" in med and write_factor:
        wb = med["WRITE_SIZE"] * 1024.0 * write_factor
        out.append(("HBM write bytes", "%.4g" % wb,
                    "WRITE_SIZE KiB x 1024 x copy calibration %.4f" % write_factor))
    if rb is not None and wb is not None and args.algo_bytes:
        out.append(("traffic / algorithmic bytes", "%.3f" % ((rb + wb) / args.algo_bytes),
                    "(read + write) / %d compulsory bytes" % args.algo_bytes))
        if dur_ns:
            out.append(("HBM rate", "%.1f GB/s" % ((rb + wb) / dur_ns),
                        "(read + write) / dispatch duration"))
    return out


def counters(args) -> int:
    if len(args.command) != len(args.pmc):
        raise SystemExit("one --command per --pmc file (%d vs %d)" % (len(args.command),
                                                                     len(args.pmc)))
    vals, durs = _load(args.pmc)
    kernels = []
    for (k, _c) in vals:
        if args.kernel in k and k not in kernels:
            kernels.append(k)
    if not kernels:
        raise SystemExit("no dispatch of a kernel matching %r" % args.kernel)
    ff = _copy_factor(vals, "FETCH_SIZE", args.copy_kernel, args.copy_bytes)
    wf = _copy_factor(vals, "WRITE_SIZE", args.copy_kernel, args.copy_bytes)
    lines = ["# rocprofv3 counters: %s" % args.title, "",
             "Commands (run from the repository root on one MI355X; each `--pmc` pass is a "
             "run of its own):", ""]
    lines += ["    " + c for c in args.command]
    lines += ["", "Values are medians over the dispatches of each kernel (a counter's "
              "instances summed per dispatch)."]
    for k in kernels:
        med = _median_by_counter(vals, k)
        # the duration comes from the pass that read GRBM_GUI_ACTIVE, else the first
        grbm = {d[0] for d in vals.get((k, "GRBM_GUI_ACTIVE"), {})}
        timed = [p for p in args.pmc if (k, p) in durs]
        timed = [p for p in timed if p in grbm] or timed
        dur = statistics.median(durs[(k, timed[0])].values()) if timed else None
        ndisp = max(len(per) for (kk, _c), per in vals.items() if kk == k)
        lines += ["", "## `%s`" % _short(k, 160), "", "%d dispatches per pass." % ndisp, "",
                  "| counter | median per dispatch |", "|---|---|"]
        for c in sorted(med):
            lines.append("| %s | %.0f |" % (c, med[c]))
        rows = derived(med, args, dur, ff, wf)
        if rows:
            lines += ["", "| derived | value | from |", "|---|---|---|"]
            lines += ["| %s | %s | %s |" % r for r in rows]
    if args.note:
        lines += ["", args.note]
    with open(args.out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))
    return 0


# ---------------------------------------------------------------- traffic

def _calibrated(path: str, counter: str, kernel_substr: str, copy_substr: str,
                copy_bytes: int):
    vals, _ = _load([path])
    per_kernel = {k: statistics.median(per.values()) for (k, c), per in vals.items()
                  if c == counter and kernel_substr in k}
    factor = _copy_factor(vals, counter, copy_substr, copy_bytes)
    if not per_kernel or factor is None:
        raise SystemExit("%s: need both library (%d) and copy dispatches" %
                         (path, len(per_kernel)))
    kib = sum(per_kernel.values())
    copy_kib = copy_bytes / 1024.0 / factor
    copy_name = next(k for (k, c) in vals if c == counter and copy_substr in k.lower())
    return {"counter_kib": kib, "factor": factor, "bytes": kib * 1024.0 * factor,
            "copy_kernel": copy_name, "copy_counter_kib": copy_kib,
            "kernels": sorted(per_kernel)}


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
        "kernels": rd["kernels"],
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
    s.add_argument("--title", default="")
    s.add_argument("--kernel", default=LIB_KERNELS)
    s.add_argument("--bytes", type=int, default=0, help="algorithmic bytes per launch")
    s.add_argument("--flop", type=int, default=0, help="FLOP per launch")
    t = sub.add_parser("traffic")
    t.add_argument("--fetch", required=True)
    t.add_argument("--write", required=True)
    t.add_argument("--copy-bytes", type=int, required=True)
    t.add_argument("--kernel", default=LIB_KERNELS)
    t.add_argument("--copy-kernel", default="copy")
    t.add_argument("--command", required=True)
    t.add_argument("--out", required=True)
    c = sub.add_parser("counters")
    c.add_argument("--pmc", action="append", required=True)
    c.add_argument("--command", action="append", required=True)
    c.add_argument("--title", required=True)
    c.add_argument("--out", required=True)
    c.add_argument("--kernel", default=LIB_KERNELS)
    c.add_argument("--copy-kernel", default="copy")
    c.add_argument("--copy-bytes", type=int, default=0)
    c.add_argument("--flop", type=int, default=0, help="closed-form FLOP (or OP) per launch")
    c.add_argument("--mfma-flop", type=int, default=0, help="FLOP per MFMA instruction")
    c.add_argument("--algo-bytes", type=int, default=0, help="compulsory bytes per launch")
    c.add_argument("--cus", type=int, default=256)
    c.add_argument("--simds", type=int, default=4)
    c.add_argument("--xcds", type=int, default=8)
    c.add_argument("--note", default="")
    args = ap.parse_args(argv)
    return {"stats": stats, "traffic": traffic, "counters": counters}[args.cmd](args)


if __name__ == "__main__":
    sys.exit(main())
