"""Summaries of rocprofv3 output for the training-step kernels.

    python -m differentiable_rasterization_amd.profiling stats <run_kernel_stats.csv>
    python -m differentiable_rasterization_amd.profiling traffic --fetch <fetch counter csv>
        --write <write counter csv> --kernel k_raster_bwd --copy-bytes <bytes read by the copy kernel>
    python -m differentiable_rasterization_amd.profiling counters <counter csv> [kernel ...]
    python -m differentiable_rasterization_amd.profiling rates --fetch <fetch counter csv>
        --write <write counter csv> --stats <run_kernel_stats.csv> --copy-bytes <bytes> [kernel ...]

`traffic` turns FETCH_SIZE / WRITE_SIZE (KiB per dispatch, as rocprofv3 reports them)
into HBM bytes per launch of one kernel.  Each counter is first divided by what it
reads, per byte, for a plain copy kernel of known size in the same run (an elementwise
multiply by a scalar over float32 buffers: it reads and writes `--copy-bytes` bytes), so
that the figure is in bytes the copy kernel would have moved.  It also prints the hash of
the sources the kernel is built from: a stored traffic figure is valid only while that
hash is unchanged (`kernel_source_hash`).
"""
from __future__ import annotations

import argparse
import collections
import csv
import hashlib
import os
import re
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")

# sources each profiled kernel is compiled from (its own file, the headers it includes,
# and the build flags)
KERNEL_SOURCES = {
    "k_raster_bwd": ["raster_bwd.hip", "raster_walk.h", "raster.h", "kernels.h", "common.h"],
    "k_raster_fwd": ["raster_fwd.hip", "raster_walk.h", "raster.h", "common.h"],
    "k_raster_fused_l1": ["raster_fused.hip", "raster_walk.h", "raster.h", "kernels.h", "common.h"],
    "k_adam": ["optim.hip", "kernels.h", "common.h"],
    "k_grad_adam": ["project.hip", "raster.h", "kernels.h", "common.h"],
    "k_grad_adam_batch": ["project.hip", "raster.h", "kernels.h", "common.h"],
}

COPY_KERNEL = re.compile(r"vectorized_elementwise_kernel.*MulFunctor")


def kernel_source_hash(kernel: str) -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel] + ["../build.py"]:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def short_name(name: str) -> str:
    name = name.replace("(anonymous namespace)::", "").replace("void ", "")
    return name.split("(")[0].strip()


def _rows(path):
    with open(path, newline="") as fh:
        return list(csv.DictReader(fh))


def stats(path: str) -> str:
    rows = _rows(path)
    out = [f"{'kernel':60s} {'calls':>6s} {'total_us':>10s} {'avg_us':>9s} {'min_us':>9s} {'max_us':>9s} {'pct':>6s}"]
    for r in sorted(rows, key=lambda r: -float(r["TotalDurationNs"])):
        out.append(f"{short_name(r['Name'])[:60]:60s} {int(r['Calls']):6d} {float(r['TotalDurationNs']) / 1e3:10.1f} "
                   f"{float(r['AverageNs']) / 1e3:9.2f} {float(r['MinNs']) / 1e3:9.2f} {float(r['MaxNs']) / 1e3:9.2f} "
                   f"{float(r['Percentage']):6.2f}")
    return "\n".join(out)


def counter_means(path: str):
    """{kernel: {counter: mean value per dispatch}} and dispatch counts."""
    acc = collections.defaultdict(lambda: collections.defaultdict(list))
    for r in _rows(path):
        acc[r["Kernel_Name"]][r["Counter_Name"]].append(float(r["Counter_Value"]))
    means = {k: {c: sum(v) / len(v) for c, v in d.items()} for k, d in acc.items()}
    counts = {k: max(len(v) for v in d.values()) for k, d in acc.items()}
    return means, counts


def _find(means, pattern):
    hits = [k for k in means if re.search(pattern, k)]
    if not hits:
        raise SystemExit(f"no kernel matching {pattern!r} in the counter file")
    return hits


def traffic(fetch_csv: str, write_csv: str, kernel: str, copy_bytes: int) -> str:
    fm, fc = counter_means(fetch_csv)
    wm, wc = counter_means(write_csv)
    cf = _find(fm, COPY_KERNEL.pattern)
    cw = _find(wm, COPY_KERNEL.pattern)
    f_copy = sum(fm[k]["FETCH_SIZE"] for k in cf) / len(cf) * 1024.0 / copy_bytes
    w_copy = sum(wm[k]["WRITE_SIZE"] for k in cw) / len(cw) * 1024.0 / copy_bytes
    ks = [k for k in _find(fm, r"\b" + re.escape(kernel) + r"\b")]
    lines = [f"copy kernel: FETCH_SIZE reads {f_copy:.4f} x and WRITE_SIZE {w_copy:.4f} x the bytes it moves "
             f"({copy_bytes} B each way)"]
    for k in ks:
        kw = [x for x in wm if short_name(x) == short_name(k)]
        fetch = fm[k]["FETCH_SIZE"] * 1024.0
        write = (sum(wm[x]["WRITE_SIZE"] for x in kw) / len(kw) * 1024.0) if kw else float("nan")
        lines.append(f"kernel {short_name(k)}: dispatches {fc[k]}; FETCH_SIZE {fetch / 1024:.0f} KiB, WRITE_SIZE "
                     f"{write / 1024:.0f} KiB per dispatch")
        lines.append(f"  traffic_bytes_per_launch {fetch / f_copy + write / w_copy:.0f}  "
                     f"(read {fetch / f_copy:.0f} + written {write / w_copy:.0f}, copy-normalised)")
    lines.append(f"source_hash {kernel} {kernel_source_hash(kernel)}")
    return "\n".join(lines)


def rates(fetch_csv: str, write_csv: str, stats_csv: str, copy_bytes: int, kernels) -> str:
    """Copy-normalised HBM bytes per dispatch of every kernel (or those matching the
    patterns), with its mean duration from a kernel-trace run of the same command: the
    achieved rate is counted bytes over time, all dispatches of a kernel together."""
    fm, fc = counter_means(fetch_csv)
    wm, _ = counter_means(write_csv)
    f_copy = sum(fm[k]["FETCH_SIZE"] for k in _find(fm, COPY_KERNEL.pattern)) / len(_find(fm, COPY_KERNEL.pattern))
    w_copy = sum(wm[k]["WRITE_SIZE"] for k in _find(wm, COPY_KERNEL.pattern)) / len(_find(wm, COPY_KERNEL.pattern))
    f_copy *= 1024.0 / copy_bytes
    w_copy *= 1024.0 / copy_bytes
    dur = {short_name(r["Name"]): (int(r["Calls"]), float(r["AverageNs"])) for r in _rows(stats_csv)}
    wsum = collections.defaultdict(list)
    for k, c in wm.items():
        wsum[short_name(k)].append(c["WRITE_SIZE"])
    lines = [f"copy kernel: FETCH_SIZE reads {f_copy:.4f} x and WRITE_SIZE {w_copy:.4f} x the bytes it moves "
             f"({copy_bytes} B each way)",
             f"{'kernel':40s} {'dispatches':>10s} {'read_MB':>10s} {'write_MB':>10s} {'avg_us':>9s} {'GB/s':>8s}"]
    for k in sorted(fm, key=lambda x: -fm[x]["FETCH_SIZE"]):
        name = short_name(k)
        if name not in dur or COPY_KERNEL.search(k):
            continue
        if kernels and not any(re.search(p, name) for p in kernels):
            continue
        rd = fm[k]["FETCH_SIZE"] * 1024.0 / f_copy
        wr = sum(wsum[name]) / len(wsum[name]) * 1024.0 / w_copy if wsum.get(name) else 0.0
        calls, avg_ns = dur[name]
        lines.append(f"{name[:40]:40s} {fc[k]:10d} {rd / 1e6:10.1f} {wr / 1e6:10.1f} {avg_ns / 1e3:9.2f} "
                     f"{(rd + wr) / avg_ns:8.1f}")
    return "\n".join(lines)


def counters(path: str, kernels) -> str:
    means, counts = counter_means(path)
    out = []
    for k in sorted(means, key=short_name):
        if kernels and not any(re.search(p, k) for p in kernels):
            continue
        c = means[k]
        out.append(f"{short_name(k)}  (dispatches {counts[k]})")
        for n in sorted(c):
            out.append(f"    {n:28s} {c[n]:16.1f}")
        if "SQ_ACTIVE_INST_VALU" in c and "GRBM_GUI_ACTIVE" in c:
            # SQ_ACTIVE_INST_VALU sums over the CUs; GRBM_GUI_ACTIVE over the 8 XCDs
            busy = 100.0 * c["SQ_ACTIVE_INST_VALU"] / 256.0 / (c["GRBM_GUI_ACTIVE"] / 8.0)
            out.append(f"    VALU busy % (SQ_ACTIVE_INST_VALU / 256 CU / GRBM_GUI_ACTIVE per XCD) {busy:.1f}")
        if "SQ_INSTS_VALU" in c and "GRBM_GUI_ACTIVE" in c:
            # a CU's four SIMDs together issue at most one wave64 VALU instruction per cycle
            issue = 100.0 * c["SQ_INSTS_VALU"] / 256.0 / (c["GRBM_GUI_ACTIVE"] / 8.0)
            out.append(f"    VALU issue % (SQ_INSTS_VALU / 256 CU / GRBM_GUI_ACTIVE per XCD) {issue:.1f}")
        if "SQ_INSTS_VALU" in c and "SQ_WAVES" in c and c["SQ_WAVES"] > 0:
            out.append(f"    VALU instructions per wave {c['SQ_INSTS_VALU'] / c['SQ_WAVES']:.1f}")
    return "\n".join(out)


def read_stored_traffic(path: str, kernel: str):
    """Traffic bytes per launch from a stored summary, or None if the file is missing or
    the kernel's sources changed since the counters were taken."""
    try:
        text = open(path).read()
    except OSError:
        return None
    m = re.search(r"source_hash " + re.escape(kernel) + r" ([0-9a-f]+)", text)
    t = re.search(r"traffic_bytes_per_launch (\d+)", text)
    if not m or not t or m.group(1) != kernel_source_hash(kernel):
        return None
    return int(t.group(1))


def main(argv=None):
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    a = sub.add_parser("stats")
    a.add_argument("csv")
    b = sub.add_parser("traffic")
    b.add_argument("--fetch", required=True)
    b.add_argument("--write", required=True)
    b.add_argument("--kernel", required=True)
    b.add_argument("--copy-bytes", type=int, required=True)
    r = sub.add_parser("rates")
    r.add_argument("--fetch", required=True)
    r.add_argument("--write", required=True)
    r.add_argument("--stats", required=True)
    r.add_argument("--copy-bytes", type=int, required=True)
    r.add_argument("kernels", nargs="*")
    c = sub.add_parser("counters")
    c.add_argument("csv")
    c.add_argument("kernels", nargs="*")
    args = ap.parse_args(argv)
    if args.cmd == "stats":
        print(stats(args.csv))
    elif args.cmd == "traffic":
        print(traffic(args.fetch, args.write, args.kernel, args.copy_bytes))
    elif args.cmd == "rates":
        print(rates(args.fetch, args.write, args.stats, args.copy_bytes, args.kernels))
    else:
        print(counters(args.csv, args.kernels))


if __name__ == "__main__":
    sys.exit(main())
