"""Summaries of rocprofv3 output for the committed performance record.

    python -m fp8_w8a8_quantized_token_amd.profiling stats <kernel_stats.csv> --command "<cmd>" [--out file.md]
    python -m fp8_w8a8_quantized_token_amd.profiling traffic <fetch counter csv> <write counter csv>
        --kernel <substring> --command "<cmd>" [--group GRID=BYTES[:LABEL] ...] [--out file.md] [--json file.json]
    python -m fp8_w8a8_quantized_token_amd.profiling runs <kernel_trace.csv> --kernel <substring>
        [--after <substring>] [--min-run N]
    python -m fp8_w8a8_quantized_token_amd.profiling counters <counter_collection.csv> --kernel <substring>
        --command "<cmd>" [--group GRID=FLOP[:LABEL] ...] [--out file.md] [--json file.json]

``stats`` renders rocprofv3's ``--kernel-trace --stats`` table (calls, average and
min/max duration per kernel). ``traffic`` turns ``--pmc FETCH_SIZE`` and
``--pmc WRITE_SIZE`` runs into HBM bytes per launch of one kernel, for each launch
shape (grid size) separately, with the traffic / algorithmic ratio, scaled by what
the same counters read for a plain 1 GiB device copy in the same run (the bench's
``--copy-calibration`` launches), and records the SHA-256 of the GEMM source the
counters were taken on so that stale figures are not reported as current.
``runs`` reads ``--kernel-trace`` records and lists the stretches in which one kernel
ran back to back (at least ``--min-run`` launches in a row), or, with ``--after``,
the stretches in which it directly followed another kernel each time (a two-kernel
step), with the kernel's mean and median duration and the mean idle gap before it:
so one region of a benchmark can be matched with its kernel-trace durations.
``counters`` summarises any other ``--pmc`` run per launch shape (the matrix-core busy
share, the MFMA flop issued, LDS and memory-pipeline counters).
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
XCDS = 8      # MI355X: XCDs, one GRBM each
SIMDS = 1024  # 256 CUs x 4 SIMDs


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


def _by_grid(per, kernel):
    """{grid_size: [counter values]} over the launches whose name contains `kernel`."""
    out = {}
    for name, v in per.items():
        if kernel in name:
            for g, x in v:
                out.setdefault(g, []).append(x)
    return out


def traffic(fetch_csv, write_csv, kernel, sources=GEMM_SOURCES, groups=None):
    """HBM bytes per launch of the kernels matching `kernel`, one record per launch shape.

    Launches are grouped by their grid size (work-items), since one kernel serves several
    shapes in a run (activations and weights, for instance) and a median across shapes
    would describe none of them. `groups` maps grid sizes to (algorithmic bytes, label)
    for the traffic / algorithmic ratio; the first entry is the primary record whose
    figures are also given at the top level."""
    fetch = _per_kernel(fetch_csv, "FETCH_SIZE")
    write = _per_kernel(write_csv, "WRITE_SIZE")
    cal_fetch = _calibration(fetch)
    cal_write = _calibration(write)
    f_by, w_by = _by_grid(fetch, kernel), _by_grid(write, kernel)
    if not f_by or not w_by:
        raise ValueError(f"kernel {kernel!r} not found in the counter runs")
    fetch_scale = CALIBRATION_BYTES / (cal_fetch * 1024)
    write_scale = CALIBRATION_BYTES / (cal_write * 1024)
    groups = dict(groups or {})
    order = [g for g in groups if g in f_by and g in w_by] + sorted(g for g in f_by if g in w_by and g not in groups)
    if not order:
        raise ValueError("no launch shape has both counters")
    recs = []
    for g in order:
        fk, wk = statistics.median(f_by[g]), statistics.median(w_by[g])
        rec = {"grid_size": g, "launches": len(f_by[g]), "fetch_kib_raw_median": fk, "write_kib_raw_median": wk,
               "fetch_bytes_per_launch": fk * 1024 * fetch_scale, "write_bytes_per_launch": wk * 1024 * write_scale}
        rec["hbm_bytes_per_launch"] = rec["fetch_bytes_per_launch"] + rec["write_bytes_per_launch"]
        if g in groups:
            algo, label = groups[g]
            rec.update(label=label, algorithmic_bytes_per_launch=algo,
                       traffic_over_algorithmic=rec["hbm_bytes_per_launch"] / algo)
        recs.append(rec)
    primary = recs[0]
    return {
        "kernel": kernel,
        "groups": recs,
        "launches": primary["launches"],
        "grid_size": primary["grid_size"],
        "fetch_kib_raw_median": primary["fetch_kib_raw_median"],
        "write_kib_raw_median": primary["write_kib_raw_median"],
        "calibration_copy_fetch_kib": cal_fetch,
        "calibration_copy_write_kib": cal_write,
        "fetch_scale": fetch_scale,
        "write_scale": write_scale,
        "fetch_bytes_per_launch": primary["fetch_bytes_per_launch"],
        "write_bytes_per_launch": primary["write_bytes_per_launch"],
        "hbm_bytes_per_launch": primary["hbm_bytes_per_launch"],
        "source": [os.path.relpath(p, os.path.dirname(PKG_DIR)) for p in sources],
        "source_sha256": sources_sha256(sources),
        # the FP8 GEMM's sources at measurement (the bench reports the traffic only while they match)
        "gemm_source_sha256": sources_sha256(GEMM_SOURCES),
    }


def traffic_markdown(t, command):
    out = ["# rocprofv3 HBM traffic (FETCH_SIZE / WRITE_SIZE)", "", f"Command: `{command}`", "",
           f"Kernel filter: `{t['kernel']}`; launches grouped by grid size (work-items), medians per group.", "",
           "Scale: the counters' reading for a plain 1 GiB device copy in the same run",
           f"(FETCH {t['calibration_copy_fetch_kib']:.0f} KiB, WRITE {t['calibration_copy_write_kib']:.0f} KiB per 1 GiB)",
           f"gives fetch x{t['fetch_scale']:.3f}, write x{t['write_scale']:.3f}.", "",
           "| launch shape | grid size | launches | FETCH raw KiB | WRITE raw KiB | fetched MB | written MB | "
           "HBM MB | algorithmic MB | traffic / algorithmic |",
           "|---|---|---|---|---|---|---|---|---|---|"]
    for r in t["groups"]:
        algo = r.get("algorithmic_bytes_per_launch")
        out.append(f"| {r.get('label', '-')} | {r['grid_size']} | {r['launches']} | {r['fetch_kib_raw_median']:.0f} | "
                   f"{r['write_kib_raw_median']:.0f} | {r['fetch_bytes_per_launch'] / 1e6:.2f} | "
                   f"{r['write_bytes_per_launch'] / 1e6:.2f} | {r['hbm_bytes_per_launch'] / 1e6:.2f} | "
                   + (f"{algo / 1e6:.2f} | {r['traffic_over_algorithmic']:.2f} |" if algo else "- | - |"))
    src = t["source"] if isinstance(t["source"], str) else " + ".join(t["source"])
    out += ["", f"Kernel source `{src}` SHA-256 at measurement: `{t['source_sha256']}`"]
    return "\n".join(out) + "\n"


def _group_for(groups, name, grid):
    """The (value, label) of the first group whose key matches a launch: a key is a grid
    size, or (kernel-name substring, grid size) where two kernels share a grid size."""
    for key, val in groups.items():
        if isinstance(key, tuple):
            if key[1] == grid and key[0] in name:
                return key, val
        elif key == grid:
            return key, val
    return None, None


def counters(csv_path, kernel, groups=None):
    """Median per launch of every counter in a ``--pmc`` run, for the kernels matching
    `kernel`, one record per (kernel, grid size); `groups` maps grid sizes, or
    (kernel-name substring, grid size) pairs, to (algorithmic flop, label).

    rocprofv3 sums a counter over all its hardware instances, so GRBM_GUI_ACTIVE (one
    per XCD) reads the XCD count times the kernel's busy cycles, and
    SQ_VALU_MFMA_BUSY_CYCLES is the sum over every SIMD. Derived figures:
      mfma_busy      SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / xcds * simds): the
                     share of SIMD cycles in which the matrix core was busy;
      mfma_flop      SQ_INSTS_VALU_MFMA_MOPS_F8 * 512: the matrix flop issued (to compare
                     with the algorithmic 2 M N K; tails padded to whole tiles add to it);
      gui_clock_ghz  GRBM_GUI_ACTIVE / xcds / duration (when the CSV has timestamps)."""
    per = {}
    for r in csv.DictReader(open(csv_path)):
        if kernel not in r["Kernel_Name"]:
            continue
        g = (r["Kernel_Name"], int(r["Grid_Size"]))
        d = per.setdefault(g, {"names": set(), "counters": {}, "dur": {}})
        d["names"].add(r["Kernel_Name"])
        d["counters"].setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
        if r.get("Start_Timestamp") and r.get("End_Timestamp"):
            d["dur"][r.get("Dispatch_Id") or r.get("Correlation_Id")] = (
                int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e9
    if not per:
        raise ValueError(f"kernel {kernel!r} not found in {csv_path}")
    groups = dict(groups or {})
    keys = list(groups)
    matched = {g: _group_for(groups, g[0], g[1]) for g in per}
    # launches named by a group first, in the groups' order, then the rest
    order = sorted(per, key=lambda g: (keys.index(matched[g][0]) if matched[g][0] is not None else len(keys),
                                       g[1], g[0]))
    out = []
    for g in order:
        d = per[g]
        med = {c: statistics.median(v) for c, v in d["counters"].items()}
        rec = {"grid_size": g[1], "kernel": g[0],
               "launches": max(len(v) for v in d["counters"].values()), "counters": med}
        if d["dur"]:
            rec["duration_us"] = statistics.median(d["dur"].values()) * 1e6
        if matched[g][0] is not None:
            rec["algorithmic_flop"], rec["label"] = matched[g][1]
        gui = med.get("GRBM_GUI_ACTIVE")
        if gui and "SQ_VALU_MFMA_BUSY_CYCLES" in med:
            rec["mfma_busy"] = med["SQ_VALU_MFMA_BUSY_CYCLES"] / (gui / XCDS * SIMDS)
        if "SQ_INSTS_VALU_MFMA_MOPS_F8" in med:
            rec["mfma_flop"] = med["SQ_INSTS_VALU_MFMA_MOPS_F8"] * 512
        if gui and rec.get("duration_us"):
            rec["gui_clock_ghz"] = gui / XCDS / (rec["duration_us"] * 1e-6) / 1e9
        out.append(rec)
    return out


def counters_markdown(recs, command):
    names = sorted({c for r in recs for c in r["counters"]})
    out = ["# rocprofv3 counters per launch", "", f"Command: `{command}`", "",
           "Medians per launch, grouped by grid size (work-items). rocprofv3 sums each counter over its hardware",
           f"instances: GRBM_GUI_ACTIVE over the {XCDS} XCDs, the SQ counters over all CUs / SIMDs.", ""]
    for r in recs:
        out += [f"## {r.get('label', 'grid ' + str(r['grid_size']))}: `{_short(r['kernel'])}`", "",
                f"grid size {r['grid_size']}, {r['launches']} launches" +
                (f", median duration {r['duration_us']:.2f} us" if "duration_us" in r else ""), "",
                "| counter | median per launch |", "|---|---|"]
        out += [f"| {c} | {r['counters'][c]:.6g} |" for c in names if c in r["counters"]]
        if "mfma_busy" in r:
            out.append(f"| matrix-core busy share of SIMD cycles (MFMA_BUSY / (GUI_ACTIVE/{XCDS} x {SIMDS})) "
                       f"| {r['mfma_busy']:.4f} |")
        if "mfma_flop" in r:
            out.append(f"| MFMA flop issued (MOPS_F8 x 512) | {r['mfma_flop']:.6g} |")
            if "algorithmic_flop" in r:
                out.append(f"| algorithmic flop 2MNK | {r['algorithmic_flop']:.6g} |")
        if "gui_clock_ghz" in r:
            out.append(f"| GUI-active clock (GRBM_GUI_ACTIVE/{XCDS} / duration) | {r['gui_clock_ghz']:.3f} GHz |")
        out.append("")
    return "\n".join(out)


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
    b.add_argument("--group", action="append", default=[], metavar="GRID=BYTES[:LABEL]",
                   help="algorithmic bytes per launch (and a label) of the launches with this grid size; "
                        "the first group is the record's primary figure")
    b.add_argument("--source", nargs="+", default=GEMM_SOURCES,
                   help="the kernel's source files, hashed (in this order) into the record")
    b.add_argument("--out")
    b.add_argument("--json")
    d = sub.add_parser("counters")
    d.add_argument("csv")
    d.add_argument("--kernel", required=True)
    d.add_argument("--group", action="append", default=[], metavar="[NAME@]GRID=FLOP[:LABEL]",
                   help="algorithmic flop (and a label) of the launches with this grid size, or of those "
                        "whose kernel name contains NAME and have this grid size")
    d.add_argument("--command", required=True)
    d.add_argument("--out")
    d.add_argument("--json")
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
    elif args.cmd == "counters":
        groups = {}
        for g in args.group:
            key, rest = g.split("=", 1)
            flop, _, label = rest.partition(":")
            name, at, grid = key.rpartition("@")
            groups[(name, int(grid)) if at else int(grid)] = (float(flop), label or f"grid {grid}")
        recs = counters(args.csv, args.kernel, groups)
        text = counters_markdown(recs, args.command)
        if args.json:
            with open(args.json, "w") as f:
                json.dump({"command": args.command, "records": recs}, f, indent=1)
    elif args.cmd == "runs":
        text = runs_markdown(runs(args.csv, args.kernel, args.after, args.min_run), args.kernel, args.after,
                             args.command)
    else:
        groups = {}
        for g in args.group:
            grid, rest = g.split("=", 1)
            algo, _, label = rest.partition(":")
            groups[int(grid)] = (float(algo), label or f"grid {grid}")
        t = traffic(args.fetch_csv, args.write_csv, args.kernel, args.source, groups)
        text = traffic_markdown(t, args.command)
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
