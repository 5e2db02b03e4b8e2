"""Summaries of rocprofv3 output for the profiles/ directory.

    python -m chunked_gated_recurrent_amd.profiling stats DIR [--kernel SUBSTR]
        kernel-trace statistics (calls, mean / min / max duration) from the
        *_kernel_stats.csv files rocprofv3 writes with --stats -f csv
    python -m chunked_gated_recurrent_amd.profiling trace DIR --kernel SUBSTR --last N
        duration of the last N dispatches of a kernel (the timed steps of a
        run that warms up first) from *_kernel_trace.csv: mean, median, min,
        max, and the mean gap between consecutive dispatches
    python -m chunked_gated_recurrent_amd.profiling counters DIR --kernel SUBSTR
        mean per-dispatch value of every counter in *_counter_collection.csv
    python -m chunked_gated_recurrent_amd.profiling copy [GIB]
        a plain device copy of GIB GiB (three times), the reference kernel whose
        FETCH_SIZE / WRITE_SIZE readings calibrate the HBM byte counters
    python -m chunked_gated_recurrent_amd.profiling traffic FETCH_DIR WRITE_DIR
            CAL_FETCH_DIR CAL_WRITE_DIR --kernel SUBSTR [--kernel SUBSTR ...] [--gib 1]
            [--sources GROUP] [--key NAME --into FILE]
        HBM bytes per dispatch of a kernel: each counter divided by the ratio
        counter / true bytes that the same counter shows for the copy kernel.
        With several --kernel names, the per-dispatch figures are summed: the
        bytes of one call that launches each of those kernels once. The
        record carries a sha256 of the library sources the kernels are built
        from (the files of GROUP in SOURCE_GROUPS, default all), so a later
        change to those files marks it stale; --key/--into merge it into a
        JSON file under NAME.
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import sys
from collections import defaultdict

HERE = os.path.dirname(os.path.abspath(__file__))


def _find(d, suffix):
    return sorted(glob.glob(os.path.join(d, "**", "*" + suffix), recursive=True))


def kernel_stats(d, kernel=None):
    rows = []
    for f in _find(d, "kernel_stats.csv"):
        for r in csv.DictReader(open(f)):
            if kernel and kernel not in r["Name"]:
                continue
            rows.append(dict(name=r["Name"], calls=int(r["Calls"]),
                             total_ns=float(r["TotalDurationNs"]),
                             avg_ns=float(r["AverageNs"]), min_ns=float(r["MinNs"]),
                             max_ns=float(r["MaxNs"]), pct=float(r["Percentage"])))
    return rows


def trace(d, kernel, last):
    """Durations (ns) of the last `last` dispatches whose name contains
    `kernel`, in dispatch order, and the gaps between them."""
    rows = []
    for f in _find(d, "kernel_trace.csv"):
        for r in csv.DictReader(open(f)):
            if kernel in r["Kernel_Name"]:
                rows.append((int(r["Start_Timestamp"]), int(r["End_Timestamp"])))
    rows.sort()
    rows = rows[-last:]
    dur = sorted(e - b for b, e in rows)
    gaps = [rows[i + 1][0] - rows[i][1] for i in range(len(rows) - 1)]
    n = len(dur)
    return dict(n=n, mean_ns=sum(dur) / n, median_ns=dur[n // 2], min_ns=dur[0],
                max_ns=dur[-1], mean_gap_ns=(sum(gaps) / len(gaps)) if gaps else 0.0)


def counters(d, kernel):
    """{counter: mean per dispatch} over dispatches whose name contains
    `kernel` (per-dispatch values summed over their instances first)."""
    per = defaultdict(lambda: defaultdict(float))
    for f in _find(d, "counter_collection.csv"):
        for r in csv.DictReader(open(f)):
            if kernel not in r["Kernel_Name"]:
                continue
            per[r["Counter_Name"]][(f, r["Dispatch_Id"])] += float(r["Counter_Value"])
    return {c: sum(v.values()) / len(v) for c, v in per.items() if v}, \
        {c: len(v) for c, v in per.items()}


def copy_kernel(gib=1.0):
    import torch
    n = int(gib * (1 << 30)) // 4
    a = torch.ones(n, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print("copied %d bytes three times" % (n * 4))


# The library sources each measured path is built from (host dispatch,
# shared device headers and the kernel files it launches).
_COMMON = ["gla_api.cpp", "gla_device.h", "gla_internal.h"]
SOURCE_GROUPS = {
    "forward": _COMMON + ["gla_kernels.hip", "gla_mfma.h", "gla_fwd_mfma.hip"],
    "decode": _COMMON + ["gla_kernels.hip"],
    "backward": _COMMON + ["gla_kernels.hip", "gla_mfma.h", "gla_fwd_mfma.hip",
                           "gla_bwd_mfma.hip", "gla_bwd_wide.hip"],
    "conv": _COMMON + ["gla_conv.hip"],
}


def source_sha256(files=None):
    """sha256 over source files of the HIP library (names and bytes): the
    given csrc file names, or every file. Any change to them invalidates
    recorded counter readings."""
    h = hashlib.sha256()
    d = os.path.join(HERE, "csrc")
    for name in sorted(files if files is not None else os.listdir(d)):
        with open(os.path.join(d, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read() + b"\0")
    return h.hexdigest()


def traffic(fetch_dir, write_dir, cal_fetch_dir, cal_write_dir, kernels, gib=1.0):
    if isinstance(kernels, str):
        kernels = [kernels]
    true_bytes = int(gib * (1 << 30)) // 4 * 4
    cf, _ = counters(cal_fetch_dir, "copyBuffer")
    cw, _ = counters(cal_write_dir, "copyBuffer")
    f_ratio = cf["FETCH_SIZE"] * 1024 / true_bytes
    w_ratio = cw["WRITE_SIZE"] * 1024 / true_bytes
    f_kb = w_kb = 0.0
    disp = {}
    for kname in kernels:
        f, fn = counters(fetch_dir, kname)
        w, _ = counters(write_dir, kname)
        f_kb += f["FETCH_SIZE"]
        w_kb += w["WRITE_SIZE"]
        disp[kname] = fn.get("FETCH_SIZE", 0)
    fetch = f_kb * 1024 / f_ratio
    write = w_kb * 1024 / w_ratio
    return dict(kernel=" + ".join(kernels), dispatches=disp,
                fetch_counter_kb=f_kb, write_counter_kb=w_kb,
                copy_fetch_ratio=f_ratio, copy_write_ratio=w_ratio,
                fetch_bytes=fetch, write_bytes=write, traffic_bytes=fetch + write)


def main(argv=None):
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    s = sub.add_parser("stats")
    s.add_argument("dir")
    s.add_argument("--kernel")
    tr = sub.add_parser("trace")
    tr.add_argument("dir")
    tr.add_argument("--kernel", required=True)
    tr.add_argument("--last", type=int, required=True)
    c = sub.add_parser("counters")
    c.add_argument("dir")
    c.add_argument("--kernel", required=True)
    cp = sub.add_parser("copy")
    cp.add_argument("gib", nargs="?", type=float, default=1.0)
    t = sub.add_parser("traffic")
    t.add_argument("fetch_dir")
    t.add_argument("write_dir")
    t.add_argument("cal_fetch_dir")
    t.add_argument("cal_write_dir")
    t.add_argument("--kernel", required=True, action="append")
    t.add_argument("--gib", type=float, default=1.0)
    t.add_argument("--sources", choices=sorted(SOURCE_GROUPS))
    t.add_argument("--key")
    t.add_argument("--into")
    a = ap.parse_args(argv)
    if a.cmd == "stats":
        rows = kernel_stats(a.dir, a.kernel)
        print("%-60s %7s %12s %12s %12s %6s" % ("kernel", "calls", "avg_us", "min_us", "max_us", "pct"))
        for r in sorted(rows, key=lambda r: -r["total_ns"]):
            print("%-60s %7d %12.3f %12.3f %12.3f %6.2f" % (
                r["name"][:60], r["calls"], r["avg_ns"] / 1e3, r["min_ns"] / 1e3,
                r["max_ns"] / 1e3, r["pct"]))
    elif a.cmd == "trace":
        r = trace(a.dir, a.kernel, a.last)
        print("%s: last %d dispatches  mean %.3f us  median %.3f us  min %.3f us  max %.3f us"
              "  mean gap %.3f us" % (a.kernel, r["n"], r["mean_ns"] / 1e3, r["median_ns"] / 1e3,
                                      r["min_ns"] / 1e3, r["max_ns"] / 1e3, r["mean_gap_ns"] / 1e3))
    elif a.cmd == "counters":
        vals, n = counters(a.dir, a.kernel)
        for k in sorted(vals):
            print("%-36s dispatches %4d  mean %.6g" % (k, n[k], vals[k]))
    elif a.cmd == "copy":
        copy_kernel(a.gib)
    elif a.cmd == "traffic":
        r = traffic(a.fetch_dir, a.write_dir, a.cal_fetch_dir, a.cal_write_dir, a.kernel, a.gib)
        files = SOURCE_GROUPS[a.sources] if a.sources else None
        r["source_sha256"] = source_sha256(files)
        r["source"] = ("chunked_gated_recurrent_amd/csrc/{%s}" % ",".join(files)
                       if files else "chunked_gated_recurrent_amd/csrc/*")
        if files:
            r["source_files"] = files
        print(json.dumps(r, indent=1))
        if a.key and a.into:
            db = {}
            if os.path.exists(a.into):
                with open(a.into) as f:
                    db = json.load(f)
            db[a.key] = r
            with open(a.into, "w") as f:
                json.dump(db, f, indent=1, sort_keys=True)
                f.write("\n")


if __name__ == "__main__":
    sys.exit(main())
