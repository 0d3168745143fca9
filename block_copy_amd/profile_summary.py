"""Summaries of rocprofv3 output for profiles/ (measurement only).

  python -m block_copy_amd.profile_summary trace DIR --name NAME --command CMD [--workload TEXT]
      -> markdown table of a --kernel-trace run: per kernel and launch size,
         calls and average / median / min / max duration, registers,
         scratch and LDS.
  python -m block_copy_amd.profile_summary counters --fetch DIR --write DIR --name NAME
         --fetch-command CMD --write-command CMD
      -> profiles/counters_NAME.json and .md from two --pmc runs (FETCH_SIZE,
         then WRITE_SIZE).  Both counters are in KiB per dispatch; each is
         scaled by what it reads for a plain elementwise kernel of known
         traffic in the same process (bench.py --counter-calibration: torch.neg
         over 64 MiB of int32, which reads 64 MiB and writes 64 MiB).

  python -m block_copy_amd.profile_summary bursts DIR --name NAME --command CMD [--workload TEXT]
         [--decode gemv_bf16_kernel] [--per-step 36]
      -> markdown table of a --kernel-trace run of bench.py's interference
         leg: decode steps (each run of --per-step decode kernels, first
         start to last end) and decode kernels outside every copy burst and
         overlapping the bursts of each copy configuration (copy kernels
         that overlap in time form one burst).

DIR is rocprofv3's output directory (-d); the CSV files are found below it.
"""
from __future__ import annotations

import argparse
import csv
import glob
import json
import os
import re
import statistics
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CALIB_BYTES = 64 * 1024 * 1024


def _rows(d, suffix):
    files = sorted(glob.glob(os.path.join(d, "**", f"*{suffix}"), recursive=True))
    if not files:
        raise SystemExit(f"no *{suffix} under {d}")
    out = []
    for f in files:
        with open(f, newline="") as fh:
            out += list(csv.DictReader(fh))
    return out


def _get(row, *names, default=None):
    for n in names:
        if n in row and row[n] not in ("", None):
            return row[n]
    return default


def short_name(full):
    m = re.search(r"(kvcopy_\w+?_kernel)\b", full)
    if m:
        return m.group(1)
    m = re.search(r"(kvload_\w+|\w+_kernel)\b", full)
    if m:
        return m.group(1)
    return full[:60]


def _grid(row):
    g = _get(row, "Grid_Size", "Grid_Size_X")
    return int(float(g)) if g is not None else 0


def trace(args):
    rows = _rows(args.dir, "kernel_trace.csv")
    groups = {}
    for r in rows:
        name = short_name(_get(r, "Kernel_Name", default="?"))
        dur = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3    # ns -> us
        key = (name, _grid(r))
        g = groups.setdefault(key, {"d": [], "vgpr": _get(r, "Arch_VGPR_Count", "VGPR_Count"),
                                    "scratch": _get(r, "Scratch_Size", "Private_Segment_Size"),
                                    "lds": _get(r, "LDS_Block_Size", "Group_Segment_Size"),
                                    "wg": _get(r, "Workgroup_Size", "Workgroup_Size_X")})
        g["d"].append(dur)
    print(f"# Kernel trace: {args.name}\n")
    print("Command (run from the repository root on one MI355X):\n")
    print(f"```\n{args.command}\n```\n")
    if args.workload:
        print(args.workload + "\n")
    print("Per kernel and launch size (grid in work-items); durations from the trace's start and "
          "end timestamps.\n")
    print("| kernel | grid work-items | workgroup | calls | average (us) | median (us) | min (us) | "
          "max (us) | VGPRs | scratch B | LDS B |")
    print("|---|---|---|---|---|---|---|---|---|---|---|")
    for (name, grid), g in sorted(groups.items(), key=lambda kv: (-sum(kv[1]["d"]), kv[0])):
        d = g["d"]
        print(f"| {name} | {grid} | {g['wg']} | {len(d)} | {statistics.mean(d):.1f} | "
              f"{statistics.median(d):.1f} | {min(d):.1f} | {max(d):.1f} | {g['vgpr']} | "
              f"{g['scratch']} | {g['lds']} |")


def _p99(v):
    v = sorted(v)
    return v[max(0, -(-99 * len(v) // 100) - 1)]


def bursts(args):
    rows = _rows(args.dir, "kernel_trace.csv")

    def iv(r):
        return int(r["Start_Timestamp"]), int(r["End_Timestamp"])

    dec = sorted(iv(r) for r in rows if args.decode in r["Kernel_Name"])
    per = args.per_step
    steps = [(dec[i][0], dec[i + per - 1][1]) for i in range(0, len(dec) - per + 1, per)]
    copies = []
    for r in rows:
        name = short_name(r["Kernel_Name"])
        if name.startswith("kvcopy_") and "plan" not in name:
            wg = int(float(_get(r, "Workgroup_Size", "Workgroup_Size_X", default=1)))
            copies.append((iv(r), name, _grid(r) // max(wg, 1), _get(r, "Queue_Id", default="?")))
    copies.sort()
    groups = []   # copy kernels that overlap in time form one burst
    for (s0, e0), name, wgs, q in copies:
        if groups and s0 <= groups[-1]["end"]:
            groups[-1]["end"] = max(groups[-1]["end"], e0)
            groups[-1]["k"].add((name, wgs, q))
        else:
            groups.append({"start": s0, "end": e0, "k": {(name, wgs, q)}})
    for g in groups:
        g["label"] = " + ".join(f"{n} x{w} WGs (queue {q})" for n, w, q in sorted(g["k"]))

    def owner(a, b):
        """The burst that the interval [a, b] overlaps, or None."""
        for g in groups:
            if g["start"] <= b and a <= g["end"]:
                return g["label"]
        return None

    by = {}
    for what, items in (("steps", steps), ("gemvs", dec)):
        for a, b in items:
            by.setdefault(owner(a, b), {"steps": [], "gemvs": []})[what].append((b - a) / 1e3)
    print(f"# Kernel trace: {args.name}\n")
    print("Command (run from the repository root on one MI355X):\n")
    print(f"```\n{args.command}\n```\n")
    if args.workload:
        print(args.workload + "\n")
    queues = sorted({_get(r, "Queue_Id", default="?") for r in rows if args.decode in r["Kernel_Name"]})
    print(f"{len(dec)} decode kernels ({len(steps)} steps of {per}) on queue(s) {queues}; "
          f"{len(copies)} copy kernels in {len(groups)} bursts.\n")
    print("Decode steps (first decode kernel's start to the last one's end) and decode kernels, "
          "outside every burst and overlapping the bursts of each copy configuration:\n")
    print("| where | bursts | burst length median (us) | steps | step median (us) | step p99 (us) | "
          "step max (us) | decode kernels | kernel median (us) | kernel max (us) |")
    print("|---|---|---|---|---|---|---|---|---|---|")

    def cells(v):
        return (f"{len(v)} | {statistics.median(v):.1f} | {_p99(v):.1f} | {max(v):.1f}" if v
                else "0 | — | — | —")

    labels = [None] + sorted({g["label"] for g in groups})
    for lab in labels:
        d = by.get(lab, {"steps": [], "gemvs": []})
        gl = [(g["end"] - g["start"]) / 1e3 for g in groups if g["label"] == lab]
        head = (f"| outside every burst | — | —" if lab is None else
                f"| bursts of {lab} | {len(gl)} | {statistics.median(gl):.0f}")
        gv = d["gemvs"]
        gcell = (f"{len(gv)} | {statistics.median(gv):.1f} | {max(gv):.1f}" if gv else "0 | — | —")
        print(f"{head} | {cells(d['steps'])} | {gcell} |")


def _counter(d, counter):
    rows = _rows(d, "counter_collection.csv")
    per = {}
    for r in rows:
        if _get(r, "Counter_Name") != counter:
            continue
        key = (_get(r, "Kernel_Name", default="?"), _grid(r))
        per.setdefault(key, []).append(float(r["Counter_Value"]))
    if not per:
        raise SystemExit(f"no {counter} values under {d}")
    return per


def counters(args):
    sys.path.insert(0, ROOT)
    import bench
    f, w = _counter(args.fetch, "FETCH_SIZE"), _counter(args.write, "WRITE_SIZE")

    def calib(per):
        vals = [v for (k, _), xs in per.items() if re.search(r"neg", k) for v in xs]
        if not vals:
            raise SystemExit("no calibration kernel (torch.neg) in the run: use --counter-calibration")
        return statistics.median(vals)
    cf, cw = calib(f), calib(w)
    sf, sw = CALIB_BYTES / (cf * 1024), CALIB_BYTES / (cw * 1024)
    kernels = {}
    for (full, grid), xs in f.items():
        name = short_name(full)
        if not name.startswith("kvcopy_"):
            continue
        ws = w.get((full, grid))
        if not ws:
            continue
        k = kernels.setdefault(f"{name}@{grid}", {"kernel": name, "grid_work_items": grid})
        k.update({"dispatches": len(xs), "FETCH_SIZE_KiB_median": statistics.median(xs),
                  "WRITE_SIZE_KiB_median": statistics.median(ws),
                  "fetch_bytes_per_dispatch_scaled": int(statistics.median(xs) * 1024 * sf),
                  "write_bytes_per_dispatch_scaled": int(statistics.median(ws) * 1024 * sw)})
    # bench.py looks a kernel up by name: the launch size with the most dispatches
    by_name = {}
    for k in kernels.values():
        cur = by_name.get(k["kernel"])
        if cur is None or k["dispatches"] > cur["dispatches"]:
            by_name[k["kernel"]] = k
    out = {"kernel_source_sha256": bench.kernel_source_hash(),
           "calibration": {"kernel": "torch.neg on 64 MiB int32 (reads 64 MiB, writes 64 MiB)",
                           "FETCH_SIZE_KiB": cf, "WRITE_SIZE_KiB": cw, "fetch_scale": sf,
                           "write_scale": sw},
           "commands": {"fetch": args.fetch_command, "write": args.write_command},
           "kernels": by_name, "by_grid": kernels}
    out_dir = getattr(args, "out_dir", None) or os.path.join(ROOT, "profiles")
    jpath = os.path.join(out_dir, f"counters_{args.name}.json")
    with open(jpath, "w") as fh:
        json.dump(out, fh, indent=1)
    lines = [f"# Counters: {args.name}\n",
             "Two rocprofv3 PMC passes (one counter each), run from the repository root on one "
             "MI355X:\n", "```", args.fetch_command, args.write_command, "```\n",
             "Calibration: a plain elementwise kernel of known traffic (torch.neg over 64 MiB of "
             "int32, which reads 64 MiB and writes 64 MiB) runs 5 times in the same process. It "
             f"reads FETCH_SIZE = {cf:.0f} KiB and WRITE_SIZE = {cw:.0f} KiB, so fetched bytes = "
             f"FETCH_SIZE x 1024 x {sf:.4f} and written bytes = WRITE_SIZE x 1024 x {sw:.4f}.\n",
             "| kernel | grid work-items | dispatches | FETCH_SIZE KiB | WRITE_SIZE KiB | fetched "
             "MiB (scaled) | written MiB (scaled) |", "|---|---|---|---|---|---|---|"]
    for k in sorted(kernels.values(), key=lambda k: (k["kernel"], k["grid_work_items"])):
        lines.append(f"| {k['kernel']} | {k['grid_work_items']} | {k['dispatches']} | "
                     f"{k['FETCH_SIZE_KiB_median']:.0f} | {k['WRITE_SIZE_KiB_median']:.0f} | "
                     f"{k['fetch_bytes_per_dispatch_scaled'] / 2**20:.2f} | "
                     f"{k['write_bytes_per_dispatch_scaled'] / 2**20:.2f} |")
    lines.append(f"\nKernel source sha256 at the time of the passes: `{out['kernel_source_sha256']}` "
                 "(bench.py reports `traffic` only while it matches).")
    with open(os.path.join(out_dir, f"counters_{args.name}.md"), "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print(f"wrote {jpath}")


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    sub = ap.add_subparsers(dest="what", required=True)
    t = sub.add_parser("trace")
    t.add_argument("dir")
    t.add_argument("--name", required=True)
    t.add_argument("--command", required=True)
    t.add_argument("--workload", default="")
    b = sub.add_parser("bursts")
    b.add_argument("dir")
    b.add_argument("--name", required=True)
    b.add_argument("--command", required=True)
    b.add_argument("--workload", default="")
    b.add_argument("--decode", default="gemv_bf16_kernel")
    b.add_argument("--per-step", type=int, default=36)
    c = sub.add_parser("counters")
    c.add_argument("--fetch", required=True)
    c.add_argument("--write", required=True)
    c.add_argument("--name", required=True)
    c.add_argument("--fetch-command", required=True)
    c.add_argument("--write-command", required=True)
    c.add_argument("--out-dir", default=None, help="default: profiles/")
    a = ap.parse_args()
    {"trace": trace, "bursts": bursts, "counters": counters}[a.what](a)


if __name__ == "__main__":
    main()
