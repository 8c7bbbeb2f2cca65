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
import re
import shutil
import subprocess

from .build import ROOT, source_digest

KERNELS = ("gla_seg_state", "gla_seg_scan", "gla_seg_out", "gla_fused")


def short_name(mangled: str) -> str:
    for k in KERNELS:
        if k in mangled:
            return k
    return mangled if len(mangled) <= 60 else mangled[:57] + "..."


# Library kernels whose instantiations a summary tells apart by their template arguments.
LIBRARY_KERNELS = KERNELS + ("gla_bwd_dqk", "gla_dgate_totals", "gla_dgate_apply", "gla_ds0",
                             "gla_state_copy", "swiglu_mix")


def demangle(name: str) -> str:
    """An Itanium-mangled name demangled with c++filt when it is installed and can (older ones
    cannot read _Float16, DF16_); otherwise as given."""
    if not name.startswith("_Z") or shutil.which("c++filt") is None:
        return name
    r = subprocess.run(["c++filt", name], capture_output=True, text=True)
    out = r.stdout.strip() if r.returncode == 0 else ""
    return out or name


_MANGLED_ARGS = re.compile(
    r"(?:NS0_6LaggedINS0_\d+(?P<lagged>IoF32|IoF16|IoBF16)EEE|NS0_\d+(?P<io>IoF32|IoF16|IoBF16)E)?"
    r"(?P<types>(?:DF16_|f|t)*)(?:L(?P<kind>[ib])(?P<value>\d+)E)?E")
_MANGLED_TYPES = {"DF16_": "_Float16", "f": "float", "t": "unsigned short"}


def _mangled_args(name: str, kernel: str) -> str:
    """Template arguments of one of this library's kernels read from its mangled name: the few
    forms they take (an element format, possibly Lagged<>, then float/_Float16 types, then one
    integer or boolean).  Empty for any other form."""
    at = name.find(f"{len(kernel)}{kernel}I")
    if at < 0:
        return ""
    m = _MANGLED_ARGS.match(name, at + len(str(len(kernel))) + len(kernel) + 1)
    if not m:
        return ""
    args = []
    if m.group("lagged"):
        args.append(f"Lagged<{m.group('lagged')}>")
    elif m.group("io"):
        args.append(m.group("io"))
    args += [_MANGLED_TYPES[t] for t in re.findall(r"DF16_|f|t", m.group("types"))]
    if m.group("kind") == "i":
        args.append(m.group("value"))
    elif m.group("kind") == "b":
        args.append("true" if m.group("value") == "1" else "false")
    return ", ".join(args)


def display_name(name: str) -> str:
    """A library kernel's name with its template arguments, from a (de)mangled name such as
    ``void gtr::(anonymous namespace)::gla_bwd_dqk<gtr::(anonymous namespace)::Lagged<...>, float,
    true>(...)``; other kernels as short_name gives them."""
    name = demangle(name)
    if name.startswith("_Z"):
        for k in LIBRARY_KERNELS:
            if f"{len(k)}{k}" in name:
                args = _mangled_args(name, k)
                return f"{k}<{args}>" if args else k
    for k in LIBRARY_KERNELS:
        at = name.find(k + "<")
        if at < 0:
            if k + "(" in name or name == k:
                return k
            continue
        depth, i = 0, at + len(k)
        for j in range(i, len(name)):
            depth += {"<": 1, ">": -1}.get(name[j], 0)
            if depth == 0:
                args = name[i + 1:j].replace("gtr::(anonymous namespace)::", "")
                return f"{k}<{args}>"
        break
    return short_name(name)


def _csvs(directory: str, suffix: str) -> list[str]:
    return sorted(glob.glob(os.path.join(directory, "**", f"*{suffix}"), recursive=True))


def kernel_stats(directory: str) -> list[dict]:
    rows = []
    for path in _csvs(directory, "kernel_stats.csv"):
        with open(path) as f:
            for r in csv.DictReader(f):
                rows.append({
                    "kernel": display_name(r["Name"]), "calls": int(r["Calls"]),
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
