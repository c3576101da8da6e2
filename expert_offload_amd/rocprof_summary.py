"""Summaries of rocprofv3 CSV output for the kernels of libmoe.

Two kinds of input, both written by ``rocprofv3 -f csv``:

* ``--kernel-trace --stats``: ``*_kernel_stats.csv`` (per kernel name:
  calls and durations).  The summary lists every kernel with its call count
  and average / min / max duration in microseconds.
* ``--pmc FETCH_SIZE`` and ``--pmc WRITE_SIZE`` (one run each):
  ``*_counter_collection.csv`` (one row per dispatch and counter, values in
  KiB).  Each counter's per-dispatch average for a kernel is divided by the
  ratio the same counter shows on a plain copy kernel of known size, giving
  HBM bytes per launch.

The traffic summary records a hash of the sources the kernel is built from;
:func:`traffic_bytes` returns the recorded traffic only while that hash
still matches, so a figure never outlives the kernel it was measured on.

Usage::

    python -m expert_offload_amd.rocprof_summary stats DIR --out FILE --command CMD
    python -m expert_offload_amd.rocprof_summary traffic FETCH_DIR WRITE_DIR --kernel NAME
        --calib-bytes N --out FILE --command CMD
    python -m expert_offload_amd.rocprof_summary counters DIR [DIR ...] --kernel NAME [--kernel NAME]
        --out FILE --command CMD
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import os
import re
from typing import Dict, List, Optional, Tuple

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)

# Sources each profiled kernel family is compiled from.
_DECODE = ["csrc/decode_gemv.h", "csrc/decode_ctl.h", "csrc/decode_mfma.h", "csrc/route_common.h", "csrc/ffn.h",
           "csrc/device_common.h", "csrc/moe_internal.h"]
KERNEL_SOURCES = {
    "ffn_gateup_decode": ["csrc/decode_impl.h", "csrc/decode_q8_0.hip"] + _DECODE,
    "ffn_down_decode": ["csrc/decode_impl.h", "csrc/decode_q8_0.hip"] + _DECODE,
    "prefill_gemm_kernel": ["csrc/prefill.hip", "csrc/ffn.h", "csrc/device_common.h", "csrc/moe_internal.h"],
}
# Calibration kernels, in order of preference: ROCm's device-to-device copy
# blit, then an elementwise negate (reads and writes the same byte count).
CALIB_PATTERNS = ("copyBuffer", "neg_kernel")


def _family(kernel: str) -> str:
    """The KERNEL_SOURCES entry a kernel name or name prefix belongs to."""
    for fam in KERNEL_SOURCES:
        if fam in kernel:
            return fam
    raise KeyError(f"no source list for kernel {kernel}")


def source_hash(kernel: str) -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES[kernel]:
        with open(os.path.join(PKG, rel), "rb") as f:
            h.update(rel.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def _find(d: str, suffix: str) -> str:
    hits = sorted(glob.glob(os.path.join(d, "**", f"*{suffix}"), recursive=True))
    if not hits:
        raise FileNotFoundError(f"no *{suffix} under {d}")
    return hits[0]


def _short(name: str) -> str:
    """Kernel name without return type and parameter list."""
    n = re.sub(r"^void\s+", "", name.strip())
    depth, out = 0, []
    for c in n:
        if c == "(" and depth == 0:
            break
        depth += c == "<"
        depth -= c == ">"
        out.append(c)
    return "".join(out)


def kernel_stats(d: str) -> List[Tuple[str, int, float, float, float]]:
    """(name, calls, avg_us, min_us, max_us) from a --stats run, by total time."""
    rows = []
    with open(_find(d, "kernel_stats.csv")) as f:
        for r in csv.DictReader(f):
            rows.append((_short(r["Name"]), int(r["Calls"]), float(r["AverageNs"]) / 1e3,
                         float(r["MinNs"]) / 1e3, float(r["MaxNs"]) / 1e3, float(r["TotalDurationNs"])))
    rows.sort(key=lambda r: -r[5])
    return [r[:5] for r in rows]


def counter_values(d: str, counter: str) -> Dict[str, List[float]]:
    """kernel -> the counter's value for each of its dispatches."""
    acc: Dict[str, List[float]] = {}
    with open(_find(d, "counter_collection.csv")) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] == counter:
                acc.setdefault(_short(r["Kernel_Name"]), []).append(float(r["Counter_Value"]))
    return acc


def _calib(vals: Dict[str, List[float]], pattern: str) -> Tuple[str, int, float]:
    """The calibration kernel's mean over its largest dispatches (within 10%
    of the maximum): the known-size run dwarfs other uses of the same kernel."""
    for k, v in vals.items():
        if pattern in k:
            top = [x for x in v if x >= 0.9 * max(v)]
            return k, len(top), sum(top) / len(top)
    raise KeyError(f"no {pattern} kernel in the counter output")


def _pick(vals: Dict[str, List[float]], kernel: str) -> Tuple[str, int, float]:
    for k, v in vals.items():
        if kernel in k:
            return k, len(v), sum(v) / len(v)
    raise KeyError(f"kernel {kernel} not in the counter output")


def write_stats(d: str, out: str, command: str) -> None:
    rows = kernel_stats(d)
    with open(out, "w") as f:
        f.write("rocprofv3 kernel trace summary\n")
        f.write(f"command: {command}\n\n")
        f.write(f"{'kernel':70s} {'calls':>7s} {'avg_us':>9s} {'min_us':>9s} {'max_us':>9s}\n")
        for name, calls, avg, mn, mx in rows:
            f.write(f"{name[:70]:70s} {calls:7d} {avg:9.2f} {mn:9.2f} {mx:9.2f}\n")


def write_traffic(fetch_dir: str, write_dir: str, kernel: str, calib_bytes: int, out: str, command: str) -> None:
    fetch = counter_values(fetch_dir, "FETCH_SIZE")
    write = counter_values(write_dir, "WRITE_SIZE")
    lines = []
    factors = {}
    for pat in CALIB_PATTERNS:
        cf_name, nf, cf = _calib(fetch, pat)
        cw_name, nw, cw = _calib(write, pat)
        factors[pat] = (cf * 1024.0 / calib_bytes, cw * 1024.0 / calib_bytes)
        lines.append(f"calibration {cf_name}: {calib_bytes} B read and written; FETCH_SIZE {cf:.1f} KiB "
                     f"(factor {factors[pat][0]:.4f}, {nf} dispatches), WRITE_SIZE {cw:.1f} KiB "
                     f"(factor {factors[pat][1]:.4f}, {nw} dispatches)")
    f_fac, w_fac = factors[CALIB_PATTERNS[0]]
    kf, nf, vf = _pick(fetch, kernel)
    kw, nw, vw = _pick(write, kernel)
    rd = vf * 1024.0 / f_fac
    wr = vw * 1024.0 / w_fac
    with open(out, "w") as f:
        f.write(f"rocprofv3 HBM traffic of {kernel}\n")
        f.write(f"command: {command}\n\n")
        for ln in lines:
            f.write(ln + "\n")
        f.write(f"scaled by the {CALIB_PATTERNS[0]} factors\n")
        f.write(f"{kf}: {nf} dispatches, FETCH_SIZE {vf:.1f} KiB/dispatch -> {rd:.0f} B read\n")
        f.write(f"{kw}: {nw} dispatches, WRITE_SIZE {vw:.1f} KiB/dispatch -> {wr:.0f} B written\n")
        f.write(f"traffic_bytes_per_launch: {rd + wr:.0f}\n")
        f.write(f"source_hash: {source_hash(_family(kernel))}\n")


SIMD_NUM, CU_NUM, XCD_NUM = 1024, 256, 8  # MI355X: 256 compute units of 4 SIMDs in 8 XCDs


def write_counters(dirs: List[str], kernels: List[str], out: str, command: str) -> None:
    """Per-dispatch averages of every counter collected in `dirs` (one
    rocprofv3 --pmc run each) for the kernels whose names contain one of
    `kernels`, with the derived figures the counters allow:
      cycles      = GRBM_GUI_ACTIVE / XCDs (the counter is summed over the
                    8 XCDs; the quotient matches the kernel's duration
                    times the clock)
      MFMA busy % = SQ_VALU_MFMA_BUSY_CYCLES / (cycles * SIMDs)
      VALU busy % = 4 * SQ_ACTIVE_INST_VALU / (cycles * SIMDs)
      MFMA FLOP   = SQ_INSTS_VALU_MFMA_MOPS_BF16 * 512
      L2 hit %    = TCC_HIT / (TCC_HIT + TCC_MISS)
    (MI355X: 1024 SIMDs in 8 XCDs)."""
    per: Dict[str, Dict[str, List[float]]] = {}
    for d in dirs:
        with open(_find(d, "counter_collection.csv")) as f:
            for r in csv.DictReader(f):
                name = _short(r["Kernel_Name"])
                if not any(k in name for k in kernels):
                    continue
                per.setdefault(name, {}).setdefault((d, r["Counter_Name"]), []).append(float(r["Counter_Value"]))
    with open(out, "w") as f:
        f.write("rocprofv3 counters per dispatch\n")
        f.write(f"command: {command}\n\n")
        for name in sorted(per):
            f.write(f"{name}\n")
            avg: Dict[str, float] = {}
            for (d, c), v in sorted(per[name].items()):
                a = sum(v) / len(v)
                key = c if c != "GRBM_GUI_ACTIVE" else f"GRBM_GUI_ACTIVE[{os.path.basename(d.rstrip('/'))}]"
                avg[key] = a
                f.write(f"  {key:58s} {a:18.1f}   ({len(v)} dispatches)\n")

            def gui(counter):
                for d, c in per[name]:
                    if c == counter:
                        g = per[name].get((d, "GRBM_GUI_ACTIVE"))
                        return sum(g) / len(g) / XCD_NUM if g else None
                return None
            for c in ("SQ_VALU_MFMA_BUSY_CYCLES", "SQ_ACTIVE_INST_VALU", "SQ_WAIT_ANY"):
                if c in avg and gui(c):
                    f.write(f"  cycles (GRBM_GUI_ACTIVE / {XCD_NUM}) in the {c} run: {gui(c):.0f}\n")
                    break
            if "SQ_VALU_MFMA_BUSY_CYCLES" in avg and gui("SQ_VALU_MFMA_BUSY_CYCLES"):
                f.write(f"  MFMA busy: {100 * avg['SQ_VALU_MFMA_BUSY_CYCLES'] / (gui('SQ_VALU_MFMA_BUSY_CYCLES') * SIMD_NUM):.1f}%\n")
            if "SQ_ACTIVE_INST_VALU" in avg and gui("SQ_ACTIVE_INST_VALU"):
                f.write(f"  VALU busy: {100 * 4 * avg['SQ_ACTIVE_INST_VALU'] / (gui('SQ_ACTIVE_INST_VALU') * SIMD_NUM):.1f}%\n")
            if "SQ_INSTS_VALU_MFMA_MOPS_BF16" in avg:
                f.write(f"  bf16 MFMA FLOP per dispatch: {avg['SQ_INSTS_VALU_MFMA_MOPS_BF16'] * 512:.4g}\n")
            if "TCC_HIT_sum" in avg and "TCC_MISS_sum" in avg:
                h, m = avg["TCC_HIT_sum"], avg["TCC_MISS_sum"]
                f.write(f"  L2 hit rate: {100 * h / max(h + m, 1):.1f}%\n")
            f.write("\n")


def traffic_bytes(kernel: str, path: str) -> Optional[float]:
    """Recorded HBM bytes per launch, or None if absent or the sources changed."""
    if kernel not in KERNEL_SOURCES or not os.path.exists(path):
        return None
    vals = {}
    with open(path) as f:
        for line in f:
            if ":" in line:
                k, v = line.split(":", 1)
                vals[k.strip()] = v.strip()
    if vals.get("source_hash") != source_hash(kernel) or "traffic_bytes_per_launch" not in vals:
        return None
    return float(vals["traffic_bytes_per_launch"])


def main() -> None:
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    sub = p.add_subparsers(dest="what", required=True)
    s = sub.add_parser("stats")
    s.add_argument("dir")
    s.add_argument("--out", required=True)
    s.add_argument("--command", required=True)
    t = sub.add_parser("traffic")
    t.add_argument("fetch_dir")
    t.add_argument("write_dir")
    t.add_argument("--kernel", required=True)
    t.add_argument("--calib-bytes", type=int, required=True)
    t.add_argument("--out", required=True)
    t.add_argument("--command", required=True)
    c = sub.add_parser("counters")
    c.add_argument("dirs", nargs="+")
    c.add_argument("--kernel", action="append", required=True)
    c.add_argument("--out", required=True)
    c.add_argument("--command", required=True)
    a = p.parse_args()
    if a.what == "stats":
        write_stats(a.dir, a.out, a.command)
    elif a.what == "counters":
        write_counters(a.dirs, a.kernel, a.out, a.command)
    else:
        write_traffic(a.fetch_dir, a.write_dir, a.kernel, a.calib_bytes, a.out, a.command)


if __name__ == "__main__":
    main()
