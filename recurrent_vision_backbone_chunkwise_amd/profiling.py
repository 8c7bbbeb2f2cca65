"""Summaries of rocprofv3 output for this library's kernels.

    python -m recurrent_vision_backbone_chunkwise_amd.profiling stats DIR --command "..." [--out F]
        per-kernel launch statistics from a ``rocprofv3 --kernel-trace --stats``
        output directory, as a short text table headed by the command;

    python -m recurrent_vision_backbone_chunkwise_amd.profiling traffic \\
        --fetch DIR --write DIR --copy-fetch DIR --copy-write DIR --copy-bytes N \\
        --workload NAME --commands "..." [--table profiles/traffic.json]
        HBM-side bytes per launch of each kernel from ``--pmc FETCH_SIZE`` and
        ``--pmc WRITE_SIZE`` runs (KiB per dispatch), each scaled by what the
        same counter reads, per byte, for a plain device copy of N bytes; the
        result is stored with a digest of the kernel sources.
"""
from __future__ import annotations

import argparse
import collections
import csv
import glob
import json
import os

from .build import ROOT, source_digest

KERNELS = ("gla_seg_state", "gla_seg_scan", "gla_seg_out", "gla_fused")


def short_name(mangled: str) -> str:
    for k in KERNELS:
        if k in mangled:
            return k
    return mangled if len(mangled) <= 60 else mangled[:57] + "..."


def _csvs(directory: str, suffix: str) -> list[str]:
    return sorted(glob.glob(os.path.join(directory, "**", f"*{suffix}"), recursive=True))


def kernel_stats(directory: str) -> list[dict]:
    rows = []
    for path in _csvs(directory, "kernel_stats.csv"):
        with open(path) as f:
            for r in csv.DictReader(f):
                rows.append({
                    "kernel": short_name(r["Name"]), "calls": int(r["Calls"]),
                    "avg_us": float(r["AverageNs"]) / 1e3, "min_us": float(r["MinNs"]) / 1e3,
                    "max_us": float(r["MaxNs"]) / 1e3, "total_us": float(r["TotalDurationNs"]) / 1e3,
                    "percent": float(r["Percentage"]),
                })
    return rows


def counter_per_dispatch(directory: str, counter: str) -> dict[str, float]:
    """Mean over dispatches of a counter (summed over its per-dispatch rows), per kernel."""
    per_dispatch = collections.defaultdict(float)
    names = {}
    for path in _csvs(directory, "counter_collection.csv"):
        with open(path) as f:
            for r in csv.DictReader(f):
                if r["Counter_Name"] != counter:
                    continue
                key = (path, r["Dispatch_Id"])
                per_dispatch[key] += float(r["Counter_Value"])
                names[key] = short_name(r["Kernel_Name"])
    acc = collections.defaultdict(list)
    for key, v in per_dispatch.items():
        acc[names[key]].append(v)
    return {k: sum(v) / len(v) for k, v in acc.items()}


def portable_command(command: str) -> str:
    """The command with this checkout's absolute root written as $REPO."""
    return command.replace(os.path.abspath(ROOT) + "/", "$REPO/")


def cmd_stats(a) -> None:
    rows = kernel_stats(a.dir)
    lines = [f"# rocprofv3 kernel trace ({a.title})",
             f"# command ($REPO is the repository root): {portable_command(a.command)}",
             f"# kernel sources: {source_digest()}", "",
             f"{'kernel':60s} {'calls':>7s} {'avg us':>9s} {'min us':>9s} {'max us':>9s} {'% time':>7s}"]
    for r in sorted(rows, key=lambda r: -r["total_us"]):
        lines.append(f"{r['kernel']:60s} {r['calls']:7d} {r['avg_us']:9.3f} {r['min_us']:9.3f} "
                     f"{r['max_us']:9.3f} {r['percent']:7.2f}")
    text = "\n".join(lines) + "\n"
    print(text, end="")
    if a.out:
        with open(a.out, "w") as f:
            f.write(text)


def cmd_traffic(a) -> None:
    fetch = counter_per_dispatch(a.fetch, "FETCH_SIZE")
    write = counter_per_dispatch(a.write, "WRITE_SIZE")
    cf = counter_per_dispatch(a.copy_fetch, "FETCH_SIZE")
    cw = counter_per_dispatch(a.copy_write, "WRITE_SIZE")
    # the copy is the only non-library kernel that moves copy_bytes; take the largest reading
    copy_f = max(v for k, v in cf.items() if k not in KERNELS) * 1024.0
    copy_w = max(v for k, v in cw.items() if k not in KERNELS) * 1024.0
    scale_f, scale_w = copy_f / a.copy_bytes, copy_w / a.copy_bytes
    table = []
    if os.path.exists(a.table):
        with open(a.table) as f:
            table = json.load(f)
    digest = source_digest()
    table = [r for r in table if not (r.get("workload") == a.workload and r.get("kernel") in fetch)]
    for k in sorted(fetch):
        if k not in KERNELS:
            continue
        fb = fetch[k] * 1024.0 / scale_f
        wb = write.get(k, 0.0) * 1024.0 / scale_w
        row = {"kernel": k, "workload": a.workload, "source": digest,
               "fetch_bytes_per_launch": round(fb), "write_bytes_per_launch": round(wb),
               "hbm_bytes_per_launch": round(fb + wb),
               "copy_scale": {"fetch": round(scale_f, 4), "write": round(scale_w, 4),
                              "copy_bytes": a.copy_bytes},
               "commands": a.commands}
        table.append(row)
        print(json.dumps(row))
    os.makedirs(os.path.dirname(os.path.abspath(a.table)), exist_ok=True)
    with open(a.table, "w") as f:
        json.dump(table, f, indent=1)
        f.write("\n")


def main() -> None:
    ap = argparse.ArgumentParser(prog="python -m recurrent_vision_backbone_chunkwise_amd.profiling")
    sub = ap.add_subparsers(dest="cmd", required=True)
    s = sub.add_parser("stats")
    s.add_argument("dir")
    s.add_argument("--command", required=True)
    s.add_argument("--title", default="")
    s.add_argument("--out")
    t = sub.add_parser("traffic")
    for n in ("fetch", "write", "copy_fetch", "copy_write"):
        t.add_argument("--" + n.replace("_", "-"), required=True)
    t.add_argument("--copy-bytes", type=int, required=True)
    t.add_argument("--workload", required=True)
    t.add_argument("--commands", required=True)
    t.add_argument("--table", default=os.path.join(ROOT, "profiles", "traffic.json"))
    a = ap.parse_args()
    (cmd_stats if a.cmd == "stats" else cmd_traffic)(a)


if __name__ == "__main__":
    main()
