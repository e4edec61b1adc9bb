"""Summaries of rocprofv3 output for the committed performance record.

    python -m fp8_w8a8_quantized_token_amd.profiling stats <kernel_stats.csv> --command "<cmd>" [--out file.md]
    python -m fp8_w8a8_quantized_token_amd.profiling traffic <fetch counter csv> <write counter csv>
        --kernel <substring> --command "<cmd>" [--out file.md] [--json file.json]
    python -m fp8_w8a8_quantized_token_amd.profiling runs <kernel_trace.csv> --kernel <substring>
        [--after <substring>] [--min-run N]

``stats`` renders rocprofv3's ``--kernel-trace --stats`` table (calls, average and
min/max duration per kernel). ``traffic`` turns ``--pmc FETCH_SIZE`` and
``--pmc WRITE_SIZE`` runs into HBM bytes per launch of one kernel, scaled by what
the same counters read for a plain 1 GiB device copy in the same run (the bench's
``--copy-calibration`` launches), and records the SHA-256 of the GEMM source the
counters were taken on so that stale figures are not reported as current.
``runs`` reads ``--kernel-trace`` records and lists the stretches in which one kernel
ran back to back (at least ``--min-run`` launches in a row), or, with ``--after``,
the stretches in which it directly followed another kernel each time (a two-kernel
step), with the kernel's mean and median duration and the mean idle gap before it:
so one region of a benchmark can be matched with its kernel-trace durations.
"""

import argparse
import csv
import hashlib
import json
import os
import statistics
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
# the FP8 GEMM kernel's sources: the kernel and the building blocks it includes
GEMM_SOURCES = [os.path.join(PKG_DIR, "csrc", "gemm_fp8.hip"), os.path.join(PKG_DIR, "csrc", "gemm_common.h")]


def sources_sha256(paths):
    """SHA-256 over the files' bytes, in the order given."""
    h = hashlib.sha256()
    for p in paths:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()
CALIBRATION_BYTES = 1 << 30  # the bench's copy calibration moves 1 GiB per launch


def _short(name, width=90):
    name = name.replace("fp8w8a8::(anonymous namespace)::", "")
    return name if len(name) <= width else name[: width - 3] + "..."


def stats_markdown(path, command):
    rows = list(csv.DictReader(open(path)))
    out = ["# rocprofv3 kernel statistics", "", f"Command: `{command}`", "",
           "| kernel | calls | avg us | min us | max us | share % |", "|---|---|---|---|---|---|"]
    for r in rows:
        out.append(f"| `{_short(r['Name'])}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                   f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | {float(r['Percentage']):.1f} |")
    return "\n".join(out) + "\n"


def _per_kernel(path, counter):
    per = {}
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] != counter:
            continue
        per.setdefault(r["Kernel_Name"], []).append((int(r["Grid_Size"]), float(r["Counter_Value"])))
    return per


def _calibration(per):
    """KiB reported per 1 GiB device copy (the largest-grid copy launches)."""
    vals = []
    for name, v in per.items():
        if "copyBuffer" in name or "copy" in name.lower():
            big = [x for g, x in v if x > 100_000]  # > ~100 MiB: the 1 GiB calibration copies
            vals += big
    if not vals:
        raise ValueError("no calibration copy found in the counter run")
    return statistics.median(vals)


def traffic(fetch_csv, write_csv, kernel, sources=GEMM_SOURCES):
    fetch = _per_kernel(fetch_csv, "FETCH_SIZE")
    write = _per_kernel(write_csv, "WRITE_SIZE")
    cal_fetch = _calibration(fetch)
    cal_write = _calibration(write)
    f_vals = [x for name, v in fetch.items() if kernel in name for _, x in v]
    w_vals = [x for name, v in write.items() if kernel in name for _, x in v]
    if not f_vals or not w_vals:
        raise ValueError(f"kernel {kernel!r} not found in the counter runs")
    fetch_scale = CALIBRATION_BYTES / (cal_fetch * 1024)
    write_scale = CALIBRATION_BYTES / (cal_write * 1024)
    fetch_bytes = statistics.median(f_vals) * 1024 * fetch_scale
    write_bytes = statistics.median(w_vals) * 1024 * write_scale
    return {
        "kernel": kernel,
        "launches": len(f_vals),
        "fetch_kib_raw_median": statistics.median(f_vals),
        "write_kib_raw_median": statistics.median(w_vals),
        "calibration_copy_fetch_kib": cal_fetch,
        "calibration_copy_write_kib": cal_write,
        "fetch_scale": fetch_scale,
        "write_scale": write_scale,
        "fetch_bytes_per_launch": fetch_bytes,
        "write_bytes_per_launch": write_bytes,
        "hbm_bytes_per_launch": fetch_bytes + write_bytes,
        "source": [os.path.relpath(p, os.path.dirname(PKG_DIR)) for p in sources],
        "source_sha256": sources_sha256(sources),
        # the FP8 GEMM's sources at measurement (the bench reports the traffic only while they match)
        "gemm_source_sha256": sources_sha256(GEMM_SOURCES),
    }


def traffic_markdown(t, command, algorithmic=None):
    out = ["# rocprofv3 HBM traffic (FETCH_SIZE / WRITE_SIZE)", "", f"Command: `{command}`", "",
           f"Kernel filter: `{t['kernel']}` ({t['launches']} launches, medians)", "",
           "Scale: the counters' reading for a plain 1 GiB device copy in the same run",
           f"(FETCH {t['calibration_copy_fetch_kib']:.0f} KiB, WRITE {t['calibration_copy_write_kib']:.0f} KiB per 1 GiB)",
           f"gives fetch x{t['fetch_scale']:.3f}, write x{t['write_scale']:.3f}.", "",
           "| quantity | value |", "|---|---|",
           f"| FETCH_SIZE raw (KiB / launch) | {t['fetch_kib_raw_median']:.0f} |",
           f"| WRITE_SIZE raw (KiB / launch) | {t['write_kib_raw_median']:.0f} |",
           f"| fetched bytes / launch (scaled) | {t['fetch_bytes_per_launch'] / 1e6:.2f} MB |",
           f"| written bytes / launch (scaled) | {t['write_bytes_per_launch'] / 1e6:.2f} MB |",
           f"| HBM bytes / launch | {t['hbm_bytes_per_launch'] / 1e6:.2f} MB |"]
    if algorithmic:
        out.append(f"| algorithmic bytes / launch | {algorithmic / 1e6:.2f} MB |")
        out.append(f"| traffic / algorithmic | {t['hbm_bytes_per_launch'] / algorithmic:.2f} |")
    src = t["source"] if isinstance(t["source"], str) else " + ".join(t["source"])
    out += ["", f"Kernel source `{src}` SHA-256 at measurement: `{t['source_sha256']}`"]
    return "\n".join(out) + "\n"


def runs(trace_csv, kernel, after=None, min_run=100):
    rows = sorted(csv.DictReader(open(trace_csv)), key=lambda r: int(r["Start_Timestamp"]))
    names = [r["Kernel_Name"] for r in rows]
    start = [int(r["Start_Timestamp"]) for r in rows]
    end = [int(r["End_Timestamp"]) for r in rows]
    # indices of the launches of interest and the launch each one must follow
    stride = 2 if after else 1
    hits = [i for i in range(1, len(rows))
            if kernel in names[i] and (after in names[i - 1] if after else kernel in names[i - 1])]
    out, cur = [], []
    for i in hits + [None]:
        if cur and (i is None or i - cur[-1] != stride):
            if len(cur) >= min_run:
                d = [(end[k] - start[k]) / 1e3 for k in cur]
                gap = [(start[k] - end[k - 1]) / 1e3 for k in cur]
                out.append({"launches": len(cur), "mean_us": statistics.mean(d), "median_us": statistics.median(d),
                            "mean_gap_before_us": statistics.mean(gap)})
            cur = []
        if i is not None:
            cur.append(i)
    return out


def runs_markdown(found, kernel, after, command):
    what = f"`{kernel}` launches each directly after `{after}`" if after else f"`{kernel}` launches back to back"
    out = [f"Stretches of {what}:", "", "| launches | mean us | median us | mean idle gap before us |",
           "|---|---|---|---|"]
    for r in found:
        out.append(f"| {r['launches']} | {r['mean_us']:.2f} | {r['median_us']:.2f} | {r['mean_gap_before_us']:.2f} |")
    return "\n".join(out) + "\n"


def main(argv=None):
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    a = sub.add_parser("stats")
    a.add_argument("csv")
    a.add_argument("--command", required=True)
    a.add_argument("--out")
    b = sub.add_parser("traffic")
    b.add_argument("fetch_csv")
    b.add_argument("write_csv")
    b.add_argument("--kernel", required=True)
    b.add_argument("--command", required=True)
    b.add_argument("--algorithmic", type=float)
    b.add_argument("--source", nargs="+", default=GEMM_SOURCES,
                   help="the kernel's source files, hashed (in this order) into the record")
    b.add_argument("--out")
    b.add_argument("--json")
    c = sub.add_parser("runs")
    c.add_argument("csv")
    c.add_argument("--kernel", required=True)
    c.add_argument("--after")
    c.add_argument("--min-run", type=int, default=100)
    c.add_argument("--command", default="")
    c.add_argument("--out")
    args = ap.parse_args(argv)
    if args.cmd == "stats":
        text = stats_markdown(args.csv, args.command)
    elif args.cmd == "runs":
        text = runs_markdown(runs(args.csv, args.kernel, args.after, args.min_run), args.kernel, args.after,
                             args.command)
    else:
        t = traffic(args.fetch_csv, args.write_csv, args.kernel, args.source)
        text = traffic_markdown(t, args.command, args.algorithmic)
        if args.json:
            with open(args.json, "w") as f:
                json.dump(dict(t, command=args.command), f, indent=1)
    if args.out:
        with open(args.out, "w") as f:
            f.write(text)
    else:
        sys.stdout.write(text)


if __name__ == "__main__":
    main()
