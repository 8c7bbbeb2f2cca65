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
        result is stored with a digest of the kernel sources;

    python -m recurrent_vision_backbone_chunkwise_amd.profiling counters --pmc DIR [DIR ...] \
        --trace DIR --workload NAME --commands "..." [--alg KERNEL=BYTES ...] [--out F]
        per-kernel hardware counters from ``--pmc`` runs (one directory per pass) as a
        short text table: MFMA utilisation and rate, time the waves spend waiting, L2
        hit rate, and the bytes L2 read and wrote past itself, sized from its request
        counts by size class, beside each kernel's algorithmic bytes.
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
LIBRARY_KERNELS = KERNELS + ("gla_bwd_dqk", "gla_dgate_apply", "gla_ds0",
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


def counter_name(mangled: str) -> str:
    """short_name, also for the other library kernels and the rocBLAS GEMMs (Tensile's Cijk_ names
    carry the macro tile after MT)."""
    for k in LIBRARY_KERNELS:
        if k in mangled:
            return k
    if mangled.startswith("Cijk_"):
        tile = mangled.split("_MT")[1].split("_")[0] if "_MT" in mangled else "?"
        return f"rocBLAS GEMM MT{tile}"
    return short_name(mangled)


def _roles(names_by_key: dict, alternate: dict[str, int]) -> dict:
    """With `alternate` = {kernel: k}: that kernel's dispatches in each file take roles 0..k-1 in
    turn (by dispatch order), and are named kernel#role."""
    out = dict(names_by_key)
    for name, k in alternate.items():
        by_file = collections.defaultdict(list)
        for key, n in names_by_key.items():
            if n == name:
                by_file[key[0]].append(key)
        for keys in by_file.values():
            for rank, key in enumerate(sorted(keys, key=lambda x: int(x[1]))):
                out[key] = f"{name}#{rank % k}"
    return out


def trace_durations(directory: str, alternate: dict[str, int] | None = None) -> dict[str, float]:
    """Mean duration (us) per kernel from a kernel trace's per-dispatch rows (with `alternate` as
    in _roles)."""
    starts = collections.defaultdict(list)
    for path in _csvs(directory, "kernel_trace.csv"):
        with open(path) as f:
            for r in csv.DictReader(f):
                starts[counter_name(r["Kernel_Name"])].append(
                    (int(r["Start_Timestamp"]), int(r["End_Timestamp"]) - int(r["Start_Timestamp"])))
    out = {}
    for name, v in starts.items():
        k = (alternate or {}).get(name, 1)
        v.sort()
        for role in range(k):
            d = [dur for i, (_, dur) in enumerate(v) if i % k == role]
            if d:
                out[name if k == 1 else f"{name}#{role}"] = sum(d) / len(d) / 1e3
    return out


def counter_rows(directories: list[str], alternate: dict[str, int] | None = None
                 ) -> dict[str, dict[str, tuple[float, float]]]:
    """For every kernel and counter in the ``--pmc`` runs under `directories`: the means over
    dispatches of the counter's sum and of its largest value over its per-dispatch rows (the rows
    are per shader engine or cache instance).  `alternate` splits a kernel by dispatch order
    (_roles), for a kernel that serves several calls in turn."""
    acc = collections.defaultdict(lambda: [0.0, float("-inf")])
    names = {}
    for directory in directories:
        for path in _csvs(directory, "counter_collection.csv"):
            with open(path) as f:
                for r in csv.DictReader(f):
                    key = (path, r["Dispatch_Id"], r["Counter_Name"])
                    v = float(r["Counter_Value"])
                    acc[key][0] += v
                    acc[key][1] = max(acc[key][1], v)
                    names[key] = counter_name(r["Kernel_Name"])
    if alternate:
        per_dispatch = _roles({(k[0], k[1]): n for k, n in names.items()}, alternate)
        names = {k: per_dispatch[(k[0], k[1])] for k in names}
    per = collections.defaultdict(lambda: collections.defaultdict(list))
    for key, (total, peak) in acc.items():
        per[names[key]][key[2]].append((total, peak))
    return {k: {c: (sum(t for t, _ in v) / len(v), sum(m for _, m in v) / len(v)) for c, v in cs.items()}
            for k, cs in per.items()}


SIMDS = 1024  # MI355X: 256 CUs x 4 SIMDs
CLOCK_HZ = 2.4e9  # MI355X peak engine clock
MFMA_PEAK = {"F16": 2.5e15, "BF16": 2.5e15, "F32": 157.3e12}  # dense flop/s per operand type


def derived_counters(c: dict[str, tuple[float, float]], avg_us: float | None, alg: float | None) -> dict:
    """Per-launch figures from one kernel's counter means (see counter_rows)."""
    def get(name, which=0):
        return c[name][which] if name in c else None

    out = {}
    busy = get("SQ_VALU_MFMA_BUSY_CYCLES")
    if busy is not None and avg_us:
        out["mfma_busy_pct"] = 100.0 * busy / (avg_us * 1e-6 * CLOCK_HZ * SIMDS)
    mops = {t: get("SQ_INSTS_VALU_MFMA_MOPS_" + t) for t in MFMA_PEAK}
    if any(m is not None for m in mops.values()):
        # one MOP is 512 flops
        flops = 512.0 * sum(m for m in mops.values() if m is not None)
        out["mfma_gflop"] = flops / 1e9
        if avg_us:
            out["mfma_tflops"] = flops / (avg_us * 1e-6) / 1e12
            peak_s = sum(512.0 * m / MFMA_PEAK[t] for t, m in mops.items() if m is not None)
            out["mfma_peak_pct"] = 100.0 * peak_s / (avg_us * 1e-6)
    wait, active = get("SQ_WAIT_INST_ANY"), get("SQ_BUSY_CYCLES")
    if wait is not None and get("SQ_WAVE_CYCLES"):
        out["wave_wait_pct"] = 100.0 * wait / get("SQ_WAVE_CYCLES")
    lds, conflict = get("SQ_INSTS_LDS"), get("SQ_LDS_BANK_CONFLICT")
    if lds and conflict is not None:
        out["lds_conflict_per_inst"] = conflict / lds
    hit, miss = get("TCC_HIT_sum"), get("TCC_MISS_sum")
    if hit is not None and miss is not None and hit + miss > 0:
        out["l2_hit_pct"] = 100.0 * hit / (hit + miss)
    r32, r64, r128 = get("TCC_EA0_RDREQ_32B_sum"), get("TCC_EA0_RDREQ_64B_sum"), get("TCC_EA0_RDREQ_128B_sum")
    if r32 is not None and r64 is not None and r128 is not None:
        out["read_bytes"] = 32.0 * r32 + 64.0 * r64 + 128.0 * r128
    wr, wr64 = get("TCC_EA0_WRREQ_sum"), get("TCC_EA0_WRREQ_64B_sum")
    if wr is not None and wr64 is not None:
        out["write_bytes"] = 64.0 * wr64 + 32.0 * (wr - wr64)
    if alg and "read_bytes" in out and "write_bytes" in out:
        out["moved_over_alg"] = (out["read_bytes"] + out["write_bytes"]) / alg
    if avg_us and "read_bytes" in out and "write_bytes" in out:
        out["moved_gbs"] = (out["read_bytes"] + out["write_bytes"]) / (avg_us * 1e-6) / 1e9
    return out


def cmd_counters(a) -> None:
    alternate = {}
    for item in a.alternate or []:
        name, k = item.rsplit("=", 1)
        alternate[name] = int(k)
    rows = counter_rows(a.pmc, alternate)
    durations = trace_durations(a.trace, alternate) if a.trace else {}
    alg = {}
    for item in a.alg or []:
        k, v = item.split("=")
        alg[k] = float(v)
    cols = [("avg us", "avg_us", "{:8.2f}"), ("MFMA busy %", "mfma_busy_pct", "{:11.2f}"),
            ("MFMA TF/s", "mfma_tflops", "{:9.1f}"), ("% MFMA peak", "mfma_peak_pct", "{:11.2f}"), ("wait %", "wave_wait_pct", "{:6.1f}"),
            ("LDS cf/inst", "lds_conflict_per_inst", "{:11.2f}"),
            ("L2 hit %", "l2_hit_pct", "{:8.1f}"), ("read MB", "read_bytes", "{:8.2f}"),
            ("write MB", "write_bytes", "{:8.2f}"), ("alg MB", "alg_bytes", "{:8.2f}"),
            ("moved/alg", "moved_over_alg", "{:9.3f}"), ("moved GB/s", "moved_gbs", "{:10.0f}")]
    mb = {"read_bytes", "write_bytes", "alg_bytes"}
    width = max([16] + [len(k) for k in rows if k.split("#")[0] in KERNELS or a.all])
    lines = [f"# rocprofv3 hardware counters ({a.workload})",
             "# commands ($REPO is the repository root):"]
    lines += [f"#   {portable_command(c)}" for c in a.commands]
    lines += [f"# kernel sources: {a.source or source_digest()}",
              "# per launch, means over dispatches; avg us from the kernel trace; MFMA busy % = "
              f"SQ_VALU_MFMA_BUSY_CYCLES over avg us x {CLOCK_HZ / 1e9:g} GHz x {SIMDS} SIMDs; MFMA TF/s = 512 "
              "flops per SQ_INSTS_VALU_MFMA_MOPS_* over avg us; % MFMA peak against the dense peak of each "
              "operand type (fp16 2.5 PFLOP/s, fp32 157.3 TFLOP/s); wait % = SQ_WAIT_INST_ANY over SQ_WAVE_CYCLES; LDS cf/inst = "
              "SQ_LDS_BANK_CONFLICT cycles per SQ_INSTS_LDS; L2 hit % = TCC_HIT over "
              "TCC_HIT + TCC_MISS; read MB = 32/64/128 x TCC_EA0_RDREQ_{32B,64B,128B}; write MB = "
              "64 x TCC_EA0_WRREQ_64B + 32 x the other TCC_EA0_WRREQ; moved = read + write", "",
              f"{'kernel':{width}s}" + "".join(f" {h:>{len(fmt.format(0))}s}" for h, _, fmt in cols)]
    for k in sorted(rows):
        if k.split("#")[0] not in KERNELS and not a.all:
            continue
        d = derived_counters(rows[k], durations.get(k), alg.get(k))
        d["avg_us"] = durations.get(k)
        d["alg_bytes"] = alg.get(k)
        cells = []
        for h, key, fmt in cols:
            v = d.get(key)
            cw = len(fmt.format(0))
            cells.append(" " + ("-".rjust(cw) if v is None else fmt.format(v / 1e6 if key in mb else v)))
        lines.append(f"{k:{width}s}" + "".join(cells))
    lines += ["", "# raw counters, means per dispatch"]
    for k in sorted(rows):
        if k.split("#")[0] in KERNELS or a.all:
            lines.append(f"{k}: " + ", ".join(f"{c} {v[0]:.0f}" for c, v in sorted(rows[k].items())))
    text = "\n".join(lines) + "\n"
    print(text, end="")
    if a.out:
        with open(a.out, "w") as f:
            f.write(text)


def portable_command(command: str) -> str:
    """The command with this checkout's absolute root written as $REPO."""
    return command.replace(os.path.abspath(ROOT) + "/", "$REPO/")


def cmd_stats(a) -> None:
    rows = kernel_stats(a.dir)
    lines = [f"# rocprofv3 kernel trace ({a.title})",
             f"# command ($REPO is the repository root): {portable_command(a.command)}",
             f"# kernel sources: {a.source or source_digest()}", "",
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
    digest = a.source or source_digest()
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
    c = sub.add_parser("counters")
    c.add_argument("--pmc", nargs="+", required=True)
    c.add_argument("--trace")
    c.add_argument("--workload", required=True)
    c.add_argument("--commands", nargs="+", required=True)
    c.add_argument("--alg", nargs="*")
    c.add_argument("--out")
    c.add_argument("--all", action="store_true", help="also list kernels that are not this library's")
    c.add_argument("--alternate", nargs="*", metavar="KERNEL=K",
                   help="split KERNEL's dispatches into K roles taken in turn (KERNEL#0 .. #K-1)")
    for sp in (s, t, c):
        sp.add_argument("--source", help="digest of the sources the run measured (the `source` that "
                        "bench.py printed); default: the sources as they are now")
    a = ap.parse_args()
    {"stats": cmd_stats, "traffic": cmd_traffic, "counters": cmd_counters}[a.cmd](a)


if __name__ == "__main__":
    main()
