"""Markdown summaries of rocprofv3 output, for the profiles kept beside the code.

    python -m bitlinear_absmean_ternarise_bit_amd.profile_summary TRACE_DIR [--pmc DIR ...] [--match TEXT]
        [--last N [--ref TEXT]]

TRACE_DIR holds the output of ``rocprofv3 --kernel-trace [--stats] -d TRACE_DIR``
(the results database, or with ``--output-format csv`` the kernel-trace CSV);
each ``--pmc DIR`` the output of one ``rocprofv3 --pmc COUNTERS ... -d DIR
--output-format csv`` run.  Prints, for every kernel (name shortened), the
number of dispatches and the average / median / minimum / maximum duration,
grouped by launch shape, and for the counter runs the per-dispatch average
of every counter for the kernels whose name contains TEXT.

--last N keeps only the timed region of a run whose warm-up came first: the
span of the last N dispatches of the reference launch (the launch shape,
among kernels whose name contains --ref TEXT, with the most total time; by
default the kernel with the most total time), extended over the dispatches
that follow it directly while their names still contain TEXT (a step made of
several launches of one kernel family).  Every dispatch that starts inside
that span is kept, whatever its kernel.
"""
from __future__ import annotations

import argparse
import csv
import glob
import os
import sqlite3
import statistics as st
from collections import defaultdict


def _short(name: str, width: int = 96) -> str:
    name = name.replace("bitlinear::(anonymous namespace)::", "").replace("void ", "", 1)
    return name if len(name) <= width else name[: width - 3] + "..."


def kernel_rows(trace_dir: str, last: int = 0, ref: str = ""):
    """(name, duration_us, grid_threads, workgroup, lds, vgpr, agpr) per dispatch, in time
    order; with last > 0 only those inside the timed region (see the module notes)."""
    rows = []
    for db in glob.glob(os.path.join(trace_dir, "**", "*results.db"), recursive=True):
        con = sqlite3.connect(db)
        for n, start, dur, gx, wx, lds, v, a in con.execute(
                "select name, start, duration, grid_x, workgroup_x, lds_size, vgpr_count, accum_vgpr_count "
                "from kernels"):
            rows.append((start, n, dur / 1000.0, gx, wx, lds, v, a))
        con.close()
    for f in glob.glob(os.path.join(trace_dir, "**", "*kernel_trace.csv"), recursive=True):
        with open(f) as fh:
            for r in csv.DictReader(fh):
                start = int(r["Start_Timestamp"])
                dur = (int(r["End_Timestamp"]) - start) / 1000.0
                rows.append((start, r["Kernel_Name"], dur, int(r.get("Grid_Size", r.get("Grid_Size_X", 0)) or 0),
                             int(r.get("Workgroup_Size", r.get("Workgroup_Size_X", 0)) or 0),
                             int(r.get("LDS_Block_Size", r.get("Lds_Size", 0)) or 0),
                             int(r.get("VGPR_Count", r.get("Arch_VGPR_Count", 0)) or 0),
                             int(r.get("Accum_VGPR_Count", 0) or 0)))
    rows.sort(key=lambda r: r[0])
    if last > 0 and rows:
        total = defaultdict(float)
        for r in rows:
            if not ref or ref in r[1]:
                total[(r[1],) + r[3:]] += r[2]
        if not ref:  # the kernel (any shape) with the most time, then its largest shape
            by_name = defaultdict(float)
            for k, v in total.items():
                by_name[k[0]] += v
            top = max(by_name, key=by_name.get)
            total = {k: v for k, v in total.items() if k[0] == top}
            ref = top
        shape = max(total, key=total.get)
        idx = [i for i, r in enumerate(rows) if (r[1],) + r[3:] == shape]
        first, end = idx[-min(last, len(idx))], idx[-1]
        while end + 1 < len(rows) and ref in rows[end + 1][1]:
            end += 1
        t0 = rows[first][0]
        t1 = rows[end][0]
        rows = [r for r in rows if t0 <= r[0] <= t1]
    return [r[1:] for r in rows]


def counter_rows(pmc_dir: str):
    """{(kernel, counter): [value per dispatch]}."""
    out = defaultdict(list)
    for f in glob.glob(os.path.join(pmc_dir, "**", "*counter_collection.csv"), recursive=True):
        with open(f) as fh:
            for r in csv.DictReader(fh):
                out[(r["Kernel_Name"], r["Counter_Name"])].append(float(r["Counter_Value"]))
    return out


def summarise(trace_dir: str, pmc_dirs=(), match: str = "", last: int = 0, ref: str = "") -> str:
    rows = kernel_rows(trace_dir, last, ref)
    lines = []
    by_name = defaultdict(list)
    by_shape = defaultdict(list)
    for n, dur, gx, wx, lds, v, a in rows:
        by_name[n].append(dur)
        by_shape[(n, gx, wx, lds, v, a)].append(dur)
    total = sum(d for ds in by_name.values() for d in ds) or 1.0
    lines.append("| kernel | calls | avg us | median us | min us | max us | % time |")
    lines.append("|---|---|---|---|---|---|---|")
    for n, ds in sorted(by_name.items(), key=lambda kv: -sum(kv[1])):
        lines.append(f"| `{_short(n)}` | {len(ds)} | {st.mean(ds):.2f} | {st.median(ds):.2f} | {min(ds):.2f} | "
                     f"{max(ds):.2f} | {100 * sum(ds) / total:.1f} |")
    lines.append("")
    lines.append("| kernel | grid threads | wg | LDS | VGPR | AGPR | launches | avg us | min us |")
    lines.append("|---|---|---|---|---|---|---|---|---|")
    for (n, gx, wx, lds, v, a), ds in sorted(by_shape.items(), key=lambda kv: -sum(kv[1])):
        lines.append(f"| `{_short(n)}` | {gx} | {wx} | {lds} | {v} | {a} | {len(ds)} | {st.mean(ds):.2f} | "
                     f"{min(ds):.2f} |")
    for d in pmc_dirs:
        cnt = counter_rows(d)
        if not cnt:
            continue
        lines.append("")
        lines.append(f"Counters of `{os.path.basename(os.path.normpath(d))}` (per dispatch):")
        lines.append("")
        lines.append("| kernel | counter | dispatches | average | min | max |")
        lines.append("|---|---|---|---|---|---|")
        for (n, c), vals in sorted(cnt.items()):
            if match and match not in n:
                continue
            lines.append(f"| `{_short(n, 72)}` | {c} | {len(vals)} | {st.mean(vals):,.1f} | {min(vals):,.1f} | "
                         f"{max(vals):,.1f} |")
    return "\n".join(lines)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("trace_dir")
    ap.add_argument("--pmc", action="append", default=[])
    ap.add_argument("--match", default="")
    ap.add_argument("--last", type=int, default=0)
    ap.add_argument("--ref", default="")
    args = ap.parse_args()
    print(summarise(args.trace_dir, args.pmc, args.match, args.last, args.ref))


if __name__ == "__main__":
    main()
