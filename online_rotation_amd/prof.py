"""Summaries of rocprofv3 output for the library's kernels.

  python -m online_rotation_amd.prof stats DIR
      per-kernel calls / average / total duration from a
      `rocprofv3 --kernel-trace --stats --output-format csv -d DIR` run.

  python -m online_rotation_amd.prof traffic FETCH_DIR WRITE_DIR --kernel NAME
         [--match SUBSTR] --read-kernel SUBSTR --write-kernel SUBSTR --calib-bytes B
         [--workload W] [--out FILE] [--command-fetch ...] [--command-write ...]
      HBM traffic per launch of kernel NAME from two `rocprofv3 --pmc FETCH_SIZE`
      and `--pmc WRITE_SIZE` runs of `bench.py --counters`.  FETCH_SIZE is
      scaled by what it reads for a kernel that reads exactly B bytes (a sum),
      WRITE_SIZE by what it reads for one that writes exactly B bytes (a fill),
      both in the same run.  Per-dispatch values are medians over the launches.
      The record carries the SHA-256 of the kernel's sources, so that a
      reader can tell when the kernel has changed since the counters were
      taken.

  python -m online_rotation_amd.prof sq DIR [DIR ...] --kernel NAME [--match SUBSTR]
         [--mfma-ops N] [--workload W] [--command CMD ...] [--out FILE]
      SQ counters of kernel NAME from one or more `rocprofv3 --pmc SQ_...`
      runs (medians per dispatch), with derived figures: matrix-core
      instructions times N ops each, the matrix pipe's busy share of the
      SIMD-cycles while the CUs were busy (SQ_VALU_MFMA_BUSY_CYCLES over
      4 x SQ_BUSY_CU_CYCLES), VALU instructions per wavefront and LDS
      bank-conflict cycles per LDS instruction.
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import os
import statistics
import sys

HERE = os.path.dirname(os.path.abspath(__file__))

# kernel name -> the sources it is built from (for the staleness hash)
_DECODE = ["csrc/gemm_decode.hip", "csrc/gemm_common.h", "csrc/rq_device.h", "csrc/split_common.h",
           "csrc/fwht_common.h"]
_QUANT = ["csrc/rotate_quant.hip", "csrc/rq_device.h", "csrc/split_common.h", "csrc/fwht_common.h"]
KERNEL_SOURCES = {
    "gemm_ra": ["csrc/gemm_ra.hip", "csrc/gemm_common.h", "csrc/rq_device.h"],
    "gemm_decode": _DECODE,
    "gemm_decode16": _DECODE,
    "gemm_decode8": ["csrc/gemm_decode8.hip", "csrc/rq_device.h"],
    "gemm_w4a4": ["csrc/gemm_w4a4.hip", "csrc/gemm_common.h", "csrc/rq_device.h"],
    "fwht4096_mfma": _QUANT,
    "split_quant": _QUANT,
    "rowlds_quant": _QUANT,
    "kron64_mfma": ["csrc/kron.hip", "csrc/rq_device.h"],
    "kron_quant": _QUANT,
    "group_quant": ["csrc/kv_quant.hip", "csrc/rq_device.h", "csrc/split_common.h"],
    "group_quant_pair": ["csrc/kv_quant.hip", "csrc/rq_device.h", "csrc/split_common.h"],
    "split_quant8": ["csrc/quant8.hip", "csrc/rq_device.h"],
    "clip_search": ["csrc/clip_search.hip", "csrc/rq_device.h"],
}


def source_hash(kernel: str) -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES[kernel]:
        with open(os.path.join(HERE, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def _rows(d: str, pattern: str):
    rows = []
    for f in sorted(glob.glob(os.path.join(d, "**", pattern), recursive=True)):
        with open(f, newline="") as fh:
            rows += list(csv.DictReader(fh))
    return rows


def kernel_stats(d: str):
    """[(name, calls, avg_ns, total_ns)] from a --stats run, longest total first."""
    out = []
    for r in _rows(d, "*kernel_stats.csv"):
        out.append((r["Name"], int(r["Calls"]), float(r["AverageNs"]), float(r["TotalDurationNs"])))
    return sorted(out, key=lambda t: -t[3])


def counter_means(d: str, counter: str):
    """{kernel name: median value per dispatch} of one counter from a --pmc run."""
    acc = {}
    for r in _rows(d, "*counter_collection.csv"):
        if r.get("Counter_Name") != counter:
            continue
        acc.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
    return {k: statistics.median(v) for k, v in acc.items()}


def _pick(means: dict, substr: str, what: str) -> float:
    hits = [k for k in means if substr in k]
    if len(hits) != 1:
        raise SystemExit(f"{what}: {len(hits)} kernels match {substr!r}: {sorted(means)}")
    return means[hits[0]]


def main(argv=None):
    ap = argparse.ArgumentParser(prog="python -m online_rotation_amd.prof")
    sub = ap.add_subparsers(dest="cmd", required=True)
    s = sub.add_parser("stats")
    s.add_argument("dir")
    t = sub.add_parser("traffic")
    t.add_argument("fetch_dir")
    t.add_argument("write_dir")
    t.add_argument("--kernel", required=True, choices=sorted(KERNEL_SOURCES))
    t.add_argument("--match", help="substring naming the kernel's instance (default: NAME<)")
    t.add_argument("--read-kernel", required=True, help="substring naming the calibration read kernel")
    t.add_argument("--write-kernel", required=True, help="substring naming the calibration write kernel")
    t.add_argument("--calib-bytes", type=int, required=True)
    t.add_argument("--workload", default="")
    t.add_argument("--command-fetch", default="")
    t.add_argument("--command-write", default="")
    t.add_argument("--out")
    q = sub.add_parser("sq")
    q.add_argument("dirs", nargs="+")
    q.add_argument("--kernel", required=True, choices=sorted(KERNEL_SOURCES))
    q.add_argument("--match", help="substring naming the kernel's instance (default: NAME<)")
    q.add_argument("--mfma-ops", type=float, default=0.0, help="ops per matrix-core instruction")
    q.add_argument("--workload", default="")
    q.add_argument("--command", action="append", default=[])
    q.add_argument("--out")
    a = ap.parse_args(argv)
    if a.cmd == "sq":
        return sq_summary(a)
    if a.cmd == "stats":
        print(f"{'kernel':<72} {'calls':>6} {'avg_us':>10} {'total_us':>11}")
        for name, calls, avg, tot in kernel_stats(a.dir):
            sys.stdout.write(f"{name[:72]:<72} {calls:>6} {avg / 1e3:>10.3f} {tot / 1e3:>11.1f}\n")
        return
    fetch = counter_means(a.fetch_dir, "FETCH_SIZE")
    write = counter_means(a.write_dir, "WRITE_SIZE")
    kf_cal = _pick(fetch, a.read_kernel, "FETCH_SIZE calibration")
    kw_cal = _pick(write, a.write_kernel, "WRITE_SIZE calibration")
    ff = a.calib_bytes / (kf_cal * 1024.0)
    fw = a.calib_bytes / (kw_cal * 1024.0)
    match = a.match or a.kernel + "<"
    kf = _pick(fetch, match, "FETCH_SIZE kernel")
    kw = _pick(write, match, "WRITE_SIZE kernel")
    fb, wb = kf * 1024.0 * ff, kw * 1024.0 * fw
    lines = [
        f"# HBM traffic per launch of {a.kernel} ({a.workload}) from rocprofv3 FETCH_SIZE / WRITE_SIZE",
        f"command_fetch: {a.command_fetch}",
        f"command_write: {a.command_write}",
        f"calibration_read_kernel: {a.read_kernel}",
        f"calibration_write_kernel: {a.write_kernel}",
        f"calibration_bytes: {a.calib_bytes}",
        f"calibration_fetch_kib: {kf_cal:.1f}",
        f"calibration_write_kib: {kw_cal:.1f}",
        f"fetch_factor: {ff:.4f}",
        f"write_factor: {fw:.4f}",
        f"kernel: {a.kernel}",
        f"instance: {match}",
        f"workload: {a.workload}",
        f"fetch_kib_per_launch: {kf:.1f}",
        f"write_kib_per_launch: {kw:.1f}",
        f"fetch_bytes_per_launch: {fb:.0f}",
        f"write_bytes_per_launch: {wb:.0f}",
        f"traffic_bytes_per_launch: {fb + wb:.0f}",
        f"source_sha256: {source_hash(a.kernel)}",
    ]
    text = "\n".join(lines) + "\n"
    if a.out:
        with open(a.out, "w") as f:
            f.write(text)
    sys.stdout.write(text)


def sq_summary(a):
    match = a.match or a.kernel + "<"
    vals = {}
    for d in a.dirs:
        names = sorted({r["Counter_Name"] for r in _rows(d, "*counter_collection.csv")})
        for c in names:
            if c.startswith("SQ_"):
                vals[c] = _pick(counter_means(d, c), match, c)
    lines = [f"# SQ counters of {a.kernel} ({a.workload}), medians per dispatch, rocprofv3 --pmc"]
    lines += [f"command: {c}" for c in a.command]
    lines += [f"kernel: {a.kernel}", f"instance: {match}", f"workload: {a.workload}"]
    lines += [f"{c}: {v:.0f}" for c, v in sorted(vals.items())]
    if a.mfma_ops and "SQ_INSTS_MFMA" in vals:
        lines.append(f"mfma_ops_per_dispatch: {vals['SQ_INSTS_MFMA'] * a.mfma_ops:.0f}")
    if "SQ_VALU_MFMA_BUSY_CYCLES" in vals and vals.get("SQ_BUSY_CU_CYCLES"):
        lines.append(f"mfma_busy_share: {vals['SQ_VALU_MFMA_BUSY_CYCLES'] / (4 * vals['SQ_BUSY_CU_CYCLES']):.3f}")
    if "SQ_INSTS_VALU" in vals and vals.get("SQ_WAVES"):
        lines.append(f"valu_insts_per_wave: {vals['SQ_INSTS_VALU'] / vals['SQ_WAVES']:.1f}")
    if "SQ_LDS_BANK_CONFLICT" in vals and vals.get("SQ_INSTS_LDS"):
        lines.append(f"lds_conflict_cycles_per_lds_inst: {vals['SQ_LDS_BANK_CONFLICT'] / vals['SQ_INSTS_LDS']:.2f}")
    lines.append(f"source_sha256: {source_hash(a.kernel)}")
    text = "\n".join(lines) + "\n"
    if a.out:
        with open(a.out, "w") as f:
            f.write(text)
    sys.stdout.write(text)


def read_traffic(path: str, kernel: str):
    """Traffic bytes per launch from a record written by `traffic`, or None
    when the record is missing, names another kernel, or predates a change
    of the kernel's sources."""
    if not os.path.exists(path):
        return None
    rec = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                rec[k.strip()] = v.strip()
    if rec.get("kernel") != kernel or rec.get("source_sha256") != source_hash(kernel):
        return None
    return float(rec["traffic_bytes_per_launch"])


if __name__ == "__main__":
    main()
