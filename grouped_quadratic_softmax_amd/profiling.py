"""Summaries of rocprofv3 output (kernel statistics and HBM byte counters).

Two uses:

* ``stats DIR``: a markdown table of the per-kernel launch statistics that
  ``rocprofv3 --kernel-trace --stats --output-format csv -d DIR`` wrote.
* ``counters DIR...``: a markdown table of per-dispatch counter medians.
* ``traffic``: HBM bytes per launch of one kernel from two counter passes
  (``--pmc FETCH_SIZE`` and ``--pmc WRITE_SIZE``, each reported in KiB per
  dispatch), each scaled by the factor that maps the same counter onto the
  known byte count of a plain device copy (``bench.py --pmc-target copy``).
  The record carries a hash of the kernel sources, so that a reader can tell
  when the figure no longer describes the code.

The parsing only reads CSV text; nothing here touches the GPU.
"""

from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import statistics
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")

# Sources whose change makes the counter figures of the prefill kernels stale.
PREFILL_SOURCES = ("oal_prefill.h", "oal_prefill_d64.hip", "oal_device.h", "oal_layout.h", "oal_internal.h")


def source_hash(files=None) -> str:
    files = PREFILL_SOURCES if files is None else files
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def _find(d: str, suffix: str) -> list[str]:
    return sorted(glob.glob(os.path.join(d, "**", "*" + suffix), recursive=True))


def kernel_stats(d: str) -> list[dict]:
    files = _find(d, "kernel_stats.csv")
    if not files:
        raise FileNotFoundError(f"no *kernel_stats.csv under {d}")
    rows = []
    for r in csv.DictReader(open(files[0])):
        rows.append({"name": r["Name"], "calls": int(r["Calls"]), "avg_us": float(r["AverageNs"]) / 1e3,
                     "min_us": float(r["MinNs"]) / 1e3, "max_us": float(r["MaxNs"]) / 1e3,
                     "total_pct": float(r.get("Percentage", "nan") or "nan")})
    rows.sort(key=lambda x: -x["avg_us"] * x["calls"])
    return rows


def counter_values(d: str, counter: str, name_has: str) -> list[float]:
    """Per-dispatch values of one counter for kernels whose name contains
    ``name_has``."""
    vals = []
    for f in _find(d, "counter_collection.csv"):
        for r in csv.DictReader(open(f)):
            if r["Counter_Name"] == counter and name_has in r["Kernel_Name"]:
                vals.append(float(r["Counter_Value"]))
    if not vals:
        raise ValueError(f"no {counter} values for kernels matching {name_has!r} under {d}")
    return vals


def short_name(n: str, width: int = 110) -> str:
    """The kernel name without its trailing parameter list (names may hold
    parentheses of their own, e.g. ``(anonymous namespace)``)."""
    n = n.replace("(anonymous namespace)::", "")
    if n.endswith(")"):
        depth = 0
        for i in range(len(n) - 1, -1, -1):
            depth += {")": 1, "(": -1}.get(n[i], 0)
            if depth == 0:
                n = n[:i] if i > 0 else n
                break
    return n if len(n) <= width else n[: width - 3] + "..."


def stats_markdown(d: str, title: str, command: str) -> str:
    lines = [f"# {title}", "", "Command (repository root, one MI355X; `cd /tmp && export TMPDIR=/tmp` first):", "",
             "```", command, "```", "", "| kernel | calls | avg us | min us | max us |", "|---|---|---|---|---|"]
    for r in kernel_stats(d):
        lines.append(f"| `{short_name(r['name'])}` | {r['calls']} | {r['avg_us']:.2f} | {r['min_us']:.2f} | "
                     f"{r['max_us']:.2f} |")
    return "\n".join(lines) + "\n"


def counter_by_kernel(d: str, counter: str, name_has: str) -> dict:
    """Median per-dispatch value of one counter for every distinct kernel
    whose name contains ``name_has``."""
    per = {}
    for f in _find(d, "counter_collection.csv"):
        for r in csv.DictReader(open(f)):
            if r["Counter_Name"] == counter and name_has in r["Kernel_Name"]:
                per.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
    if not per:
        raise ValueError(f"no {counter} values for kernels matching {name_has!r} under {d}")
    return {k: statistics.median(v) for k, v in per.items()}


def traffic_record(fetch_dir, write_dir, copy_fetch_dir, copy_write_dir, kernel, copy_bytes, commands,
                   sources=None):
    """HBM bytes of one call: the medians per dispatch of every kernel whose
    name contains ``kernel`` (a call may launch several), summed, each
    counter scaled by the copy calibration."""
    kib = 1024.0
    fetch = sum(counter_by_kernel(fetch_dir, "FETCH_SIZE", kernel).values()) * kib
    write = sum(counter_by_kernel(write_dir, "WRITE_SIZE", kernel).values()) * kib
    cfetch = statistics.median(counter_values(copy_fetch_dir, "FETCH_SIZE", "copy")) * kib
    cwrite = statistics.median(counter_values(copy_write_dir, "WRITE_SIZE", "copy")) * kib
    ff, fw = copy_bytes / cfetch, copy_bytes / cwrite
    rec = {"bytes_per_launch": fetch * ff + write * fw, "fetch_bytes": fetch * ff, "write_bytes": write * fw,
           "fetch_counter_bytes": fetch, "write_counter_bytes": write, "fetch_factor": ff, "write_factor": fw,
           "copy_bytes": copy_bytes, "kernel_match": kernel, "source_sha256": source_hash(sources),
           "commands": commands}
    if sources is not None:
        rec["sources"] = list(sources)
    return rec


def counters_markdown(dirs, kernels, title, commands) -> str:
    """Per-dispatch medians of every counter found under ``dirs`` for the
    kernels whose names contain one of ``kernels``."""
    rows = {}
    for d in dirs:
        for f in _find(d, "counter_collection.csv"):
            for r in csv.DictReader(open(f)):
                name = r["Kernel_Name"]
                if any(k in name for k in kernels):
                    rows.setdefault(short_name(name, 90), {}).setdefault(r["Counter_Name"], []).append(
                        float(r["Counter_Value"]))
    counters = sorted({c for v in rows.values() for c in v})
    lines = [f"# {title}", "", "Commands (repository root, one MI355X; `cd /tmp && export TMPDIR=/tmp` first):", "",
             "```", *commands, "```", "", "Median per dispatch.", "",
             "| kernel | dispatches | " + " | ".join(counters) + " |", "|---|---|" + "---|" * len(counters)]
    for k, v in sorted(rows.items()):
        n = max(len(x) for x in v.values())
        cells = [f"{statistics.median(v[c]):.4g}" if c in v else "" for c in counters]
        lines.append(f"| `{k}` | {n} | " + " | ".join(cells) + " |")
    return "\n".join(lines) + "\n"


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    sub = ap.add_subparsers(dest="cmd", required=True)
    s1 = sub.add_parser("stats")
    s1.add_argument("dir")
    s1.add_argument("--title", required=True)
    s1.add_argument("--command", required=True)
    s2 = sub.add_parser("traffic")
    for a in ("fetch", "write", "copy-fetch", "copy-write", "kernel", "key", "out"):
        s2.add_argument("--" + a, required=True)
    s2.add_argument("--copy-bytes", type=int, default=1 << 30)
    s2.add_argument("--commands", nargs="*", default=[])
    s2.add_argument("--sources", nargs="*", default=None,
                    help="csrc files whose change makes the record stale (default: the chunk prefill's)")
    s3 = sub.add_parser("counters")
    s3.add_argument("dirs", nargs="+")
    s3.add_argument("--kernels", nargs="+", required=True)
    s3.add_argument("--title", required=True)
    s3.add_argument("--commands", nargs="*", default=[])
    args = ap.parse_args(argv)
    if args.cmd == "stats":
        sys.stdout.write(stats_markdown(args.dir, args.title, args.command))
        return
    if args.cmd == "counters":
        sys.stdout.write(counters_markdown(args.dirs, args.kernels, args.title, args.commands))
        return
    rec = traffic_record(args.fetch, args.write, args.copy_fetch, args.copy_write, args.kernel, args.copy_bytes,
                         args.commands, args.sources)
    table = {}
    if os.path.exists(args.out):
        with open(args.out) as f:
            table = json.load(f)
    table[args.key] = rec
    with open(args.out, "w") as f:
        json.dump(table, f, indent=1, sort_keys=True)
        f.write("\n")
    print(json.dumps(rec, indent=1))


if __name__ == "__main__":
    main()
