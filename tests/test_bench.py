"""bench.py's command-line contract: one GPU only, and the fields of its JSON line."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BENCH = os.path.join(ROOT, "bench.py")


def run(*args, timeout=300):
    return subprocess.run([sys.executable, BENCH, *args], capture_output=True, text=True, timeout=timeout,
                          cwd=ROOT)


def test_more_than_one_gpu_is_refused_with_a_message():
    r = run("--gpus", "2")
    assert r.returncode == 2 and "one GPU" in r.stderr and r.stdout == ""


def test_help_lists_the_options():
    r = run("--help")
    assert r.returncode == 0
    for opt in ("--gpus", "--steps", "--warmup", "--workload", "--op"):
        assert opt in r.stdout


@pytest.mark.gpu
def test_json_line_fields():
    """A short run of the smallest workload prints one JSON line with every field of the contract."""
    r = run("--workload", "1", "--steps", "5", "--warmup", "1", "--cpu-seconds", "0.5")
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [ln for ln in r.stdout.splitlines() if ln.startswith("{")]
    assert len(lines) == 1
    d = json.loads(lines[0])
    for key, kind in (("metric", str), ("value", float), ("unit", str), ("n_gpus", int), ("steps", int),
                      ("warmup", int), ("ms_per_step", float), ("higher_is_better", bool), ("scaling", str),
                      ("dtype", str), ("data", str), ("config", dict), ("roofline", dict),
                      ("cpu_baseline", dict)):
        assert isinstance(d[key], kind), key
    assert d["n_gpus"] == 1 and d["steps"] == 5 and d["warmup"] == 1 and d["value"] > 0
    assert d["vs_baseline"] is None and d["config"]["workload"] == "grid40x40_f32_b1h2_lr"
    rl = d["roofline"]
    assert rl["bound"] in ("hbm", "mfma", "alu") and rl["unit"] in ("GB/s", "TFLOP/s")
    assert 0 < rl["achieved"] and rl["frac"] == pytest.approx(rl["achieved"] / rl["peak"], rel=1e-3)
    assert "traffic" in rl and rl["kernel_frac"] == rl["frac"]
    # the whole call, launch gaps included, cannot beat its dominant kernel
    assert 0 < rl["call_frac"] <= 1.25 * rl["kernel_frac"]
    cb = d["cpu_baseline"]
    assert cb["kind"] == "oracle" and cb["value"] > 0 and cb["cores"] >= 1 and cb["unit"] == d["unit"]
    assert cb["host_cores"] >= 1
    assert isinstance(cb["sample"], str) and cb["sample"]
    assert d["long_sequence"] is None  # only the default workload also reports the 16K round


@pytest.mark.gpu
def test_default_run_also_reports_the_long_sequence():
    r = run("--steps", "5", "--warmup", "1", "--no-cpu-baseline")
    assert r.returncode == 0, r.stderr[-2000:]
    d = json.loads([ln for ln in r.stdout.splitlines() if ln.startswith("{")][0])
    assert d["config"]["workload"] == "grid40x40_f16_b1h6_4dir" and d["cpu_baseline"] is None
    ls = d["long_sequence"]
    assert ls["workload"] == "grid128x128_f16_b1h16_4dir" and ls["value"] > 0
    assert ls["roofline"]["kernel"] in ("gla_seg_out", "gla_seg_state", "gla_fused")
    assert 0 < ls["roofline"]["frac"] < 1 and 0 < ls["roofline"]["call_frac"] <= 1.25 * ls["roofline"]["frac"]
