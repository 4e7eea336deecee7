"""Short text summaries of rocprofv3 output for profiles/ (the figures that bench.py reads and the design notes quote).

    python profile_summary.py trace  --dir D --tag w2 --json BENCH_OUT --title T --cmd C
        kernel-trace summary -> profiles/decode_step_<tag>_kernel_trace.txt
    python profile_summary.py hbm    --name N --kernel K --fetch D1 --write D2 \\
                                     --copy-fetch D3 --copy-write D4 --alg-bytes B --title T --cmd C ...
        FETCH_SIZE / WRITE_SIZE per dispatch of kernel K, scaled by a plain copy's
        reading -> profiles/<N>_counters.txt
    python profile_summary.py sq     --name N --kernel K --dir D [--dir D2 ...] --title T --cmd C ...
        SQ / derived counters per dispatch of kernel K (medians) -> profiles/<N>_counters.txt

Every summary carries bench.source_digest(): bench.py uses a summary only while the
kernel sources are the ones it was taken from.  D arguments are rocprofv3 output
directories (--output-format csv).
"""
from __future__ import annotations

import argparse
import csv
import glob
import json
import os
import statistics
import sys

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

# short names of the decode path's kernels, by a substring of the kernel's name
SHORT = [("tiny_step_kernel", "decode_step_tiny"), ("hamming_scan_query_kernel", "hamming_scan"), ("hamming_scan_group_kernel", "hamming_scan_group"),
         ("hamming_scan_kernel", "hamming_scan"), ("emit_attend", "select_attend"),
         ("lse_merge", "lse_merge"), ("encode_query", "encode_query"),
         ("encode_keys_mfma", "encode_keys"), ("read_probe", "read_probe"),
         ("gather_probe", "gather_probe")]


def short_name(name: str) -> str:
    for sub, short in SHORT:
        if sub in name:
            return short
    return "other"


def _one(d: str, suffix: str) -> str:
    hits = glob.glob(os.path.join(d, "**", f"*{suffix}"), recursive=True)
    if not hits:
        raise SystemExit(f"no *{suffix} under {d}")
    return hits[0]


def _digest() -> str:
    import bench
    return bench.source_digest()


def trace(args):
    rows = list(csv.DictReader(open(_one(args.dir, "kernel_trace.csv"))))
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    seq = [(short_name(r["Kernel_Name"]), int(r["Start_Timestamp"]), int(r["End_Timestamp"]),
            int(r["Grid_Size_X"])) for r in rows]
    info = json.loads(open(args.json).read().strip().splitlines()[-1])
    alg = (info.get("roofline") or {}).get("alg_bytes_per_launch")
    vals = {"source_digest": _digest()}
    # runs of consecutive dispatches of one kernel: bench.py launches the scan back to back
    runs, cur = [], [seq[0]]
    for x in seq[1:]:
        if x[0] == cur[-1][0]:
            cur.append(x)
        else:
            runs.append(cur)
            cur = [x]
    runs.append(cur)
    for k in ("decode_step_tiny", "hamming_scan", "select_attend", "lse_merge", "encode_query"):
        d = [(e - s) / 1e3 for n, s, e, _ in seq if n == k]
        if d:
            vals[f"{k}_all_avg_us"] = f"{statistics.mean(d):.3f}"
            vals[f"{k}_all_dispatches"] = str(len(d))
    # dispatches that start within 1 us of the previous dispatch's end (graph replays):
    # launched while the GPU was still busy, as in back-to-back execution without the
    # profiler, so they are the ones to set beside back-to-back event timing
    for k in ("hamming_scan", "select_attend", "lse_merge"):
        d = [(seq[i][2] - seq[i][1]) / 1e3 for i in range(1, len(seq))
             if seq[i][0] == k and seq[i][1] - seq[i - 1][2] < 1000]
        if d:
            vals[f"{k}_tight_avg_us"] = f"{statistics.mean(d):.3f}"
            vals[f"{k}_tight_dispatches"] = str(len(d))
    long = [r for r in runs if r[0][0] == "hamming_scan" and len(r) >= 20]
    if long:
        d = [(e - s) / 1e3 for r in long for _, s, e, _ in r]
        gaps = [(r[i][1] - r[i - 1][2]) / 1e3 for r in long for i in range(1, len(r))]
        vals["hamming_scan_back_to_back_avg_us"] = f"{statistics.mean(d):.3f}"
        vals["hamming_scan_back_to_back_dispatches"] = str(len(d))
        vals["hamming_scan_back_to_back_median_gap_us"] = f"{statistics.median(gaps):.3f}"
    if alg:
        # the read probe over exactly the scan's bytes (32 KB per 256-thread workgroup)
        grid = alg // 128
        d = [(e - s) / 1e3 for n, s, e, g in seq if n == "read_probe" and g == grid]
        if d:
            vals["read_probe_same_size_avg_us"] = f"{statistics.mean(d):.3f}"
            vals["read_probe_same_size_dispatches"] = str(len(d))
    stats = list(csv.DictReader(open(_one(args.dir, "kernel_stats.csv"))))
    out = [f"# rocprofv3 kernel statistics: {args.title}", f"# command: {args.cmd}"]
    out += [f"# {line}" for line in NOTES_TRACE]
    out += [f"{k}: {v}" for k, v in vals.items()]
    out.append("# kernel | calls | avg us | min us | max us | share of GPU time")
    for r in stats:
        out.append(f"{r['Name'][:110]} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                   f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | {float(r['Percentage']):.1f}%")
    name = args.out or f"decode_step_{args.tag}_kernel_trace.txt"
    path = os.path.join(ROOT, "profiles", name)
    open(path, "w").write("\n".join(out) + "\n")
    print(path)


NOTES_TRACE = [
    "bench.py launches the scan back to back (a run of consecutive scan dispatches) to time it,",
    "and the read probe over exactly the scan's bytes; under the profiler consecutive",
    "dispatches are separated by the gap given below, so each one starts on an idle GPU.",
    "*_all_*: every dispatch of the kernel (the step loop, the graph replays, the separate timings).",
    "*_tight_*: the dispatches that start within 1 us of the previous dispatch's end (graph replays),",
    "as launches run back to back without the profiler; bench.py's event timing is compared with these.",
]


def _per_dispatch(d: str, kernel: str):
    """{counter: [value per dispatch of kernel]} from a --pmc run (values summed over
    the counter's dimensions)."""
    rows = list(csv.DictReader(open(_one(d, "counter_collection.csv"))))
    acc = {}
    for r in rows:
        if kernel not in r["Kernel_Name"]:
            continue
        key = (r["Counter_Name"], int(r["Dispatch_Id"]))
        acc[key] = acc.get(key, 0.0) + float(r["Counter_Value"])
    out = {}
    for (c, _), v in acc.items():
        out.setdefault(c, []).append(v)
    return out


def hbm(args):
    f = _per_dispatch(args.fetch, args.kernel)["FETCH_SIZE"]
    w = _per_dispatch(args.write, args.kernel)["WRITE_SIZE"]
    cf = statistics.median(_copy_values(args.copy_fetch, "FETCH_SIZE"))
    cw = statistics.median(_copy_values(args.copy_write, "WRITE_SIZE"))
    moved = args.copy_mib * 1024.0                       # KiB moved by the copy
    fs, ws = moved / cf, moved / cw
    fm, wm = statistics.median(f), statistics.median(w)
    rd, wr = fm * fs * 1024, wm * ws * 1024
    vals = {"source_digest": _digest(), "dispatches": str(len(f)),
            "fetch_size_kib_median": f"{fm:.1f}", "write_size_kib_median": f"{wm:.1f}",
            "fetch_scale": f"{fs:.4f}", "write_scale": f"{ws:.4f}",
            "hbm_read_bytes_per_launch": f"{rd:.0f}", "hbm_write_bytes_per_launch": f"{wr:.0f}",
            "hbm_bytes_per_launch": f"{rd + wr:.0f}"}
    if args.alg_bytes:
        vals["algorithmic_bytes_per_launch"] = str(args.alg_bytes)
        vals["traffic_over_algorithmic"] = f"{(rd + wr) / args.alg_bytes:.3f}"
    out = [f"# HBM bytes per launch of {args.kernel}, {args.title}"]
    out += [f"# command: {c}" for c in args.cmd]
    out.append(f"# calibration: a plain {args.copy_mib} MiB device copy reads FETCH_SIZE {cf:.1f} KiB, "
               f"WRITE_SIZE {cw:.1f} KiB for {moved:.0f} KiB moved each way")
    out += [f"# {n}" for n in args.note]
    out += [f"{k}: {v}" for k, v in vals.items()]
    path = os.path.join(ROOT, "profiles", f"{args.name}_counters.txt")
    open(path, "w").write("\n".join(out) + "\n")
    print(path)


def _copy_values(d, counter):
    """Per-dispatch values of counter for the device copies of a `bench.py --copy-probe`
    run: the dispatches of kernels named *copy* within 10% of the largest."""
    rows = list(csv.DictReader(open(_one(d, "counter_collection.csv"))))
    acc = {}
    for r in rows:
        if r["Counter_Name"] == counter and "copy" in r["Kernel_Name"].lower():
            k = int(r["Dispatch_Id"])
            acc[k] = acc.get(k, 0.0) + float(r["Counter_Value"])
    top = max(acc.values())
    return [x for x in acc.values() if x >= 0.9 * top]


def sq(args):
    vals = {"source_digest": _digest()}
    n = None
    for d in args.dir:
        per = _per_dispatch(d, args.kernel)
        for c, v in sorted(per.items()):
            vals[f"{c}_median"] = f"{statistics.median(v):.4g}"
            n = len(v)
    vals["dispatches"] = str(n)
    out = [f"# counters per dispatch of {args.kernel}, {args.title}"]
    out += [f"# command: {c}" for c in args.cmd]
    out += [f"# {n_}" for n_ in args.note]
    out += [f"{k}: {v}" for k, v in vals.items()]
    path = os.path.join(ROOT, "profiles", f"{args.name}_counters.txt")
    open(path, "w").write("\n".join(out) + "\n")
    print(path)


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="what", required=True)
    t = sub.add_parser("trace")
    t.add_argument("--dir", required=True)
    t.add_argument("--tag", required=True)
    t.add_argument("--json", required=True, help="the profiled bench.py run's output (its JSON line)")
    t.add_argument("--title", required=True)
    t.add_argument("--cmd", required=True)
    t.add_argument("--out", default="", help="file name under profiles/ (default from --tag)")
    h = sub.add_parser("hbm")
    for a in ("--name", "--kernel", "--fetch", "--write", "--copy-fetch", "--copy-write", "--title"):
        h.add_argument(a, required=True)
    h.add_argument("--copy-mib", type=int, default=256)
    h.add_argument("--alg-bytes", type=int, default=0)
    h.add_argument("--cmd", action="append", default=[])
    h.add_argument("--note", action="append", default=[])
    s = sub.add_parser("sq")
    for a in ("--name", "--kernel", "--title"):
        s.add_argument(a, required=True)
    s.add_argument("--dir", action="append", required=True)
    s.add_argument("--cmd", action="append", default=[])
    s.add_argument("--note", action="append", default=[])
    args = ap.parse_args()
    {"trace": trace, "hbm": hbm, "sq": sq}[args.what](args)


if __name__ == "__main__":
    main()
