"""Summaries of rocprofv3 CSV output for the HTA kernels.

Three subcommands, all reading what ``rocprofv3 --output-format csv`` writes:

  stats    per-kernel call count and durations from ``*_kernel_stats.csv``,
           written as a short text table with the command that produced it.
  traffic  HBM bytes per dispatch of one kernel from two ``--pmc`` runs
           (``FETCH_SIZE``, then ``WRITE_SIZE``; KiB per dispatch), each scaled
           by the same counter's reading on a plain copy kernel whose bytes are
           known (``hbm_copy_kernel`` under ``bench.py --copy-calibration``).
           The result is JSON keyed to a digest of the kernel's source file
           (comments excluded), so a reader can tell when the kernel changed
           after the counters were taken.
  mfma     MFMA utilisation of one kernel from a ``--pmc`` run of
           SQ_VALU_MFMA_BUSY_CYCLES, SQ_BUSY_CYCLES, SQ_INSTS_MFMA and the MFMA
           op counters: busy cycles per SIMD over the kernel's active cycles
           per shader engine (MI355X: 1024 SIMDs in 32 shader engines).

Usage:
  python -m hybrid_linear_temporal_hta_amd.profiling stats CSV --out FILE --command CMD
  python -m hybrid_linear_temporal_hta_amd.profiling traffic --kernel SUBSTR \\
      --fetch DIR --write DIR --copy-fetch DIR --copy-write DIR --copy-bytes N \\
      --source FILE --out FILE --command CMD [--last N | --first N] [--grid N]
  python -m hybrid_linear_temporal_hta_amd.profiling mfma --kernel SUBSTR --pmc DIR \\
      --source FILE --out FILE --command CMD [--last N | --first N] [--grid N]
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import re
import sys

COPY_KERNEL = "hbm_copy_kernel"


def source_digest(path: str) -> str:
    """sha256 of a C/C++/HIP source with comments and blank lines removed, so
    that documentation edits do not mark counter figures as stale."""
    text = open(path, encoding="utf-8").read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    lines = [ln.rstrip() for ln in text.splitlines() if ln.strip()]
    return hashlib.sha256("\n".join(lines).encode()).hexdigest()


def _short(name: str) -> str:
    """Kernel name without argument lists of templated host types."""
    name = re.sub(r"\(anonymous namespace\)::", "", name)
    name = re.sub(r"^void ", "", name)
    i = name.find("(")
    return name[:i] if i > 0 else name


def _find(path: str, suffix: str) -> str:
    if os.path.isfile(path):
        return path
    hits = sorted(glob.glob(os.path.join(path, "**", "*" + suffix), recursive=True))
    if not hits:
        raise FileNotFoundError(f"no *{suffix} under {path}")
    return hits[0]


def kernel_stats(path: str):
    rows = []
    with open(_find(path, "kernel_stats.csv")) as f:
        for r in csv.DictReader(f):
            rows.append({"kernel": _short(r["Name"]), "calls": int(r["Calls"]),
                         "total_ns": float(r["TotalDurationNs"]), "avg_ns": float(r["AverageNs"]),
                         "min_ns": float(r["MinNs"]), "max_ns": float(r["MaxNs"]),
                         "pct": float(r["Percentage"])})
    rows.sort(key=lambda r: -r["total_ns"])
    return rows


def trace_by_grid(path: str, prefix: str = "hta::"):
    """Durations from ``*_kernel_trace.csv`` grouped by (kernel, grid size), so
    launches of one kernel on different workloads are told apart. Also the
    longest uninterrupted run of such launches (no other kernel in between, in
    dispatch order): a loop that launches only this kernel, timed alone."""
    rows = []
    with open(_find(path, "kernel_trace.csv")) as f:
        for r in csv.DictReader(f):
            rows.append((int(r["Start_Timestamp"]), _short(r["Kernel_Name"]),
                         int(r["Grid_Size_X"]) // max(1, int(r["Workgroup_Size_X"])),
                         (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3))
    rows.sort()
    groups, runs = {}, {}
    prev, cur = None, []
    for _, name, wgs, dur in rows + [(0, None, 0, 0.0)]:
        key = (name, wgs)
        if key != prev and cur:
            if len(cur) > len(runs.get(prev, [])):
                runs[prev] = cur
            cur = []
        if name is None:
            break
        prev = key
        cur.append(dur)
        if name.startswith(prefix):
            groups.setdefault(key, []).append(dur)
    out = []
    for (name, wgs), d in groups.items():
        run = runs.get((name, wgs), [])
        out.append({"kernel": name, "workgroups": wgs, "calls": len(d),
                    "avg_us": sum(d) / len(d), "min_us": min(d), "max_us": max(d),
                    "run_calls": len(run), "run_avg_us": sum(run) / len(run) if run else 0.0})
    out.sort(key=lambda r: -r["avg_us"] * r["calls"])
    return out


def counter_per_dispatch(path: str, counter: str, kernel: str, last: int = 0, grid: int = 0,
                         first: int = 0):
    """Mean over dispatches of `kernel` (substring) of one counter's value, and
    the dispatch count; with `last` (`first`), over the last (first) that many
    dispatches only;
    with `grid`, over dispatches of that grid size (work-items) only. Values of
    one dispatch spread over several rows (one per counter dimension) are
    summed first."""
    per = {}
    with open(_find(path, "counter_collection.csv")) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] != counter or kernel not in r["Kernel_Name"]:
                continue
            if grid and int(r["Grid_Size"]) != grid:
                continue
            d = int(r["Dispatch_Id"])
            per[d] = per.get(d, 0.0) + float(r["Counter_Value"])
    if not per:
        raise ValueError(f"no {counter} rows for kernel {kernel!r} in {path}")
    if last or first:
        n = last or first
        if len(per) < n:
            raise ValueError(f"{len(per)} dispatches of {kernel!r} in {path}, fewer than {n}")
        keep = sorted(per)[-last:] if last else sorted(per)[:first]
        per = {d: per[d] for d in keep}
    return sum(per.values()) / len(per), len(per)


def cmd_stats(a):
    rows = kernel_stats(a.csv)
    lines = [f"# rocprofv3 kernel statistics: {a.title}", "", "Command:", "", "    " + a.command, "",
             f"{'kernel':<58} {'calls':>6} {'avg_us':>10} {'min_us':>10} {'max_us':>10} {'pct':>6}"]
    for r in rows[:a.top]:
        lines.append(f"{r['kernel'][:58]:<58} {r['calls']:>6} {r['avg_ns'] / 1e3:>10.1f} "
                     f"{r['min_ns'] / 1e3:>10.1f} {r['max_ns'] / 1e3:>10.1f} {r['pct']:>6.2f}")
    lines += ["", "Library kernels by launch shape (from the kernel trace); run = the longest",
              "stretch of consecutive launches of that kernel and shape with no other kernel",
              "in between (a loop timing it alone):", "",
              f"{'kernel':<34} {'workgroups':>10} {'calls':>6} {'avg_us':>9} {'min_us':>9} "
              f"{'max_us':>9} {'run':>5} {'run_avg_us':>10}"]
    for r in trace_by_grid(a.csv):
        lines.append(f"{r['kernel'][:34]:<34} {r['workgroups']:>10} {r['calls']:>6} "
                     f"{r['avg_us']:>9.1f} {r['min_us']:>9.1f} {r['max_us']:>9.1f} "
                     f"{r['run_calls']:>5} {r['run_avg_us']:>10.1f}")
    text = "\n".join(lines) + "\n"
    with open(a.out, "w") as f:
        f.write(text)
    sys.stdout.write(text)


def cmd_traffic(a):
    cf, ncf = counter_per_dispatch(a.copy_fetch, "FETCH_SIZE", COPY_KERNEL)
    cw, ncw = counter_per_dispatch(a.copy_write, "WRITE_SIZE", COPY_KERNEL)
    kf, nkf = counter_per_dispatch(a.fetch, "FETCH_SIZE", a.kernel, a.last, a.grid, a.first)
    kw, nkw = counter_per_dispatch(a.write, "WRITE_SIZE", a.kernel, a.last, a.grid, a.first)
    # the copy kernel reads and writes copy_bytes each: bytes per counted KiB
    f_fetch = a.copy_bytes / cf
    f_write = a.copy_bytes / cw
    rec = {"kernel": a.kernel, "grid_work_items": a.grid or None,
           "source": os.path.relpath(a.source, os.path.dirname(a.out) + "/.."),
           "source_digest": source_digest(a.source),
           "fetch_kib_per_dispatch": kf, "write_kib_per_dispatch": kw,
           "dispatches": [nkf, nkw],
           "copy_kernel": COPY_KERNEL, "copy_bytes_per_dispatch": a.copy_bytes,
           "copy_fetch_kib": cf, "copy_write_kib": cw, "copy_dispatches": [ncf, ncw],
           "bytes_per_fetch_unit": f_fetch, "bytes_per_write_unit": f_write,
           "hbm_read_bytes_per_launch": kf * f_fetch, "hbm_write_bytes_per_launch": kw * f_write,
           "hbm_bytes_per_launch": kf * f_fetch + kw * f_write,
           "command": a.command}
    with open(a.out, "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    print(json.dumps(rec, indent=1))


SIMDS, SHADER_ENGINES = 1024, 32   # MI355X: 256 CUs x 4 SIMDs; 8 XCDs x 4 shader engines


def cmd_mfma(a):
    names = ["SQ_VALU_MFMA_BUSY_CYCLES", "SQ_BUSY_CYCLES", "SQ_INSTS_MFMA",
             "SQ_INSTS_VALU_MFMA_MOPS_BF16", "SQ_INSTS_VALU_MFMA_MOPS_F16", "SQ_INSTS_LDS",
             "SQ_LDS_BANK_CONFLICT"]
    vals, nd = {}, 0
    for c in names:
        try:
            vals[c], nd = counter_per_dispatch(a.pmc, c, a.kernel, a.last, a.grid, a.first)
        except ValueError:
            vals[c] = None
    busy, sqb = vals["SQ_VALU_MFMA_BUSY_CYCLES"], vals["SQ_BUSY_CYCLES"]
    cyc = sqb / SHADER_ENGINES if sqb else None   # active cycles of the kernel
    rec = {"kernel": a.kernel, "grid_work_items": a.grid or None,
           "source": os.path.relpath(a.source, os.path.dirname(a.out) + "/.."),
           "source_digest": source_digest(a.source), "dispatches": nd,
           "per_dispatch": vals, "active_cycles": cyc,
           "mfma_busy_frac": busy / (cyc * SIMDS) if busy is not None and cyc else None,
           "busy_cycles_per_mfma": busy / vals["SQ_INSTS_MFMA"]
           if busy and vals["SQ_INSTS_MFMA"] else None,
           "command": a.command}
    with open(a.out, "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    print(json.dumps(rec, indent=1))


def main(argv=None):
    ap = argparse.ArgumentParser(prog="python -m hybrid_linear_temporal_hta_amd.profiling")
    sub = ap.add_subparsers(dest="cmd", required=True)
    s = sub.add_parser("stats")
    s.add_argument("csv")
    s.add_argument("--out", required=True)
    s.add_argument("--command", required=True)
    s.add_argument("--title", default="")
    s.add_argument("--top", type=int, default=12)
    t = sub.add_parser("traffic")
    for k in ("kernel", "fetch", "write", "copy_fetch", "copy_write", "source", "out", "command"):
        t.add_argument("--" + k.replace("_", "-"), dest=k, required=True)
    t.add_argument("--copy-bytes", dest="copy_bytes", type=float, required=True)
    t.add_argument("--last", type=int, default=0,
                   help="only the last N dispatches of the kernel (default: all)")
    m = sub.add_parser("mfma")
    for k in ("kernel", "pmc", "source", "out", "command"):
        m.add_argument("--" + k, dest=k, required=True)
    for q in (t, m):
        q.add_argument("--grid", type=int, default=0, help="only dispatches of this grid size")
        q.add_argument("--first", type=int, default=0, help="only the first N dispatches")
    m.add_argument("--last", type=int, default=0, help="only the last N dispatches")
    a = ap.parse_args(argv)
    {"stats": cmd_stats, "traffic": cmd_traffic, "mfma": cmd_mfma}[a.cmd](a)


if __name__ == "__main__":
    main()
