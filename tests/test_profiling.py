"""The rocprofv3 summary tooling (recurrent_vision_backbone_chunkwise_amd.profiling) on synthetic
rocprofv3 CSV files (CPU)."""
import csv
import json
import subprocess
import sys

from recurrent_vision_backbone_chunkwise_amd import profiling
from recurrent_vision_backbone_chunkwise_amd.build import ROOT, source_digest

MANGLED = "_ZN3gtr12_GLOBAL__N_111gla_seg_outINS0_5IoF16EDF16_Li1EEEvNS0_6ParamsE"


def write_counters(directory, counter, rows):
    directory.mkdir(parents=True, exist_ok=True)
    with open(directory / "p_counter_collection.csv", "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        for dispatch, name, value in rows:
            w.writerow([dispatch, name, counter, value])


def test_kernel_stats_and_summary(tmp_path):
    d = tmp_path / "trace"
    d.mkdir()
    with open(d / "run_kernel_stats.csv", "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Name", "Calls", "TotalDurationNs", "AverageNs", "Percentage", "MinNs", "MaxNs"])
        w.writerow([MANGLED, 4, 20000, 5000, 80.0, 4000, 6000])
        w.writerow(["__amd_rocclr_copyBuffer", 2, 5000, 2500, 20.0, 2000, 3000])
    rows = profiling.kernel_stats(str(d))
    assert rows[0] == {"kernel": "gla_seg_out<IoF16, _Float16, 1>", "calls": 4, "avg_us": 5.0, "min_us": 4.0, "max_us": 6.0,
                       "total_us": 20.0, "percent": 80.0}
    out = tmp_path / "summary.txt"
    cmd = f"rocprofv3 --kernel-trace --stats -- python3 {ROOT}/bench.py"
    subprocess.run([sys.executable, "-m", "recurrent_vision_backbone_chunkwise_amd.profiling", "stats", str(d),
                    "--command", cmd, "--title", "t", "--out", str(out)], check=True, capture_output=True,
                   cwd=ROOT)
    text = out.read_text()
    assert "$REPO/bench.py" in text and ROOT + "/" not in text
    assert f"# kernel sources: {source_digest()}" in text
    assert text.index("gla_seg_out") < text.index("__amd_rocclr_copyBuffer")  # sorted by total time


def test_display_names_keep_template_arguments():
    name = ("void gtr::(anonymous namespace)::gla_bwd_dqk<gtr::(anonymous namespace)::Lagged<gtr::(anonymous "
            "namespace)::IoF16>, float, true>(gtr::(anonymous namespace)::Params, void*, float*, float const*, "
            "void const*)")
    assert profiling.display_name(name) == "gla_bwd_dqk<Lagged<IoF16>, float, true>"
    assert profiling.display_name("gla_seg_out") == "gla_seg_out"
    assert profiling.display_name("gtr::(anonymous namespace)::gla_state_copy(float const*, float*, long long)") == \
        "gla_state_copy"
    assert profiling.display_name(MANGLED) == "gla_seg_out<IoF16, _Float16, 1>"
    assert profiling.display_name("_ZN3gtr12_GLOBAL__N_110swiglu_mixIDF16_DF16_EEvPKT0_PKT_S7_PS5_iiiiii") == \
        "swiglu_mix<_Float16, _Float16>"
    assert profiling.display_name(
        "_ZN3gtr12_GLOBAL__N_111gla_bwd_dqkINS0_6LaggedINS0_5IoF32EEEfLb1EEEvNS0_6ParamsEPvPfPKfPKv") == \
        "gla_bwd_dqk<Lagged<IoF32>, float, true>"


def test_traffic_scaled_by_the_copy(tmp_path):
    # kernel: 2 dispatches of 3 and 5 KiB (two rows each for the first) fetched, 1 KiB written;
    # the copy of 1 MiB reads 2048 KiB on FETCH_SIZE (scale 2) and 1024 KiB on WRITE_SIZE (scale 1)
    write_counters(tmp_path / "f", "FETCH_SIZE", [(1, MANGLED, 1), (1, MANGLED, 2), (2, MANGLED, 5)])
    write_counters(tmp_path / "w", "WRITE_SIZE", [(1, MANGLED, 1), (2, MANGLED, 1)])
    write_counters(tmp_path / "cf", "FETCH_SIZE", [(1, "copy_kernel", 2048), (2, "small", 3)])
    write_counters(tmp_path / "cw", "WRITE_SIZE", [(1, "copy_kernel", 1024)])
    table = tmp_path / "traffic.json"
    table.write_text(json.dumps([{"kernel": "gla_seg_out", "workload": "wl", "source": "old"},
                                 {"kernel": "gla_seg_out", "workload": "other", "source": "keep"}]))
    subprocess.run([sys.executable, "-m", "recurrent_vision_backbone_chunkwise_amd.profiling", "traffic",
                    "--fetch", str(tmp_path / "f"), "--write", str(tmp_path / "w"),
                    "--copy-fetch", str(tmp_path / "cf"), "--copy-write", str(tmp_path / "cw"),
                    "--copy-bytes", str(1 << 20), "--workload", "wl", "--commands", "c", "--table", str(table)],
                   check=True, capture_output=True, cwd=ROOT)
    rows = json.loads(table.read_text())
    assert [r["source"] for r in rows if r["workload"] == "other"] == ["keep"]
    (row,) = [r for r in rows if r["workload"] == "wl"]
    assert row["fetch_bytes_per_launch"] == 4 * 1024 / 2  # mean of 3 and 5 KiB, halved
    assert row["write_bytes_per_launch"] == 1024
    assert row["hbm_bytes_per_launch"] == 3072
    assert row["source"] == source_digest() and row["copy_scale"]["fetch"] == 2.0


def write_multi(directory, rows):
    directory.mkdir(parents=True, exist_ok=True)
    with open(directory / "p_counter_collection.csv", "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        for row in rows:
            w.writerow(row)


def test_counter_table(tmp_path):
    # one dispatch: MFMA busy over 2 rows, GUI active per instance (largest taken), hits and
    # misses, read requests by size and writes by size
    write_multi(tmp_path / "p1", [(1, MANGLED, "SQ_VALU_MFMA_BUSY_CYCLES", 600), (1, MANGLED, "SQ_VALU_MFMA_BUSY_CYCLES", 424),
                                  (1, MANGLED, "GRBM_GUI_ACTIVE", 10), (1, MANGLED, "GRBM_GUI_ACTIVE", 4),
                                  (1, MANGLED, "SQ_INSTS_VALU_MFMA_MOPS_F16", 1000),
                                  (1, MANGLED, "SQ_WAIT_INST_ANY", 30), (1, MANGLED, "SQ_WAVE_CYCLES", 120),
                                  (1, MANGLED, "SQ_INSTS_LDS", 8), (1, MANGLED, "SQ_LDS_BANK_CONFLICT", 2)])
    write_multi(tmp_path / "p2", [(1, MANGLED, "TCC_HIT_sum", 3), (1, MANGLED, "TCC_MISS_sum", 1),
                                  (1, MANGLED, "TCC_EA0_RDREQ_sum", 10), (1, MANGLED, "TCC_EA0_RDREQ_DRAM_sum", 5)])
    write_multi(tmp_path / "p3", [(1, MANGLED, "TCC_EA0_RDREQ_32B_sum", 2), (1, MANGLED, "TCC_EA0_RDREQ_64B_sum", 3),
                                  (1, MANGLED, "TCC_EA0_RDREQ_128B_sum", 5),
                                  (1, MANGLED, "TCC_EA0_WRREQ_sum", 4), (1, MANGLED, "TCC_EA0_WRREQ_64B_sum", 3)])
    rows = profiling.counter_rows([str(tmp_path / p) for p in ("p1", "p2", "p3")])
    d = profiling.derived_counters(rows["gla_seg_out"], avg_us=2.0, alg=900.0)
    assert d["mfma_busy_pct"] == 100.0 * 1024 / (2e-6 * profiling.CLOCK_HZ * profiling.SIMDS)
    assert d["mfma_gflop"] == 512 * 1000 / 1e9 and d["mfma_tflops"] == 512 * 1000 / 2e-6 / 1e12
    assert abs(d["mfma_peak_pct"] - 100.0 * 512 * 1000 / 2.5e15 / 2e-6) < 1e-12
    assert d["lds_conflict_per_inst"] == 0.25
    assert d["wave_wait_pct"] == 25.0 and d["l2_hit_pct"] == 75.0
    assert d["read_bytes"] == 32 * 2 + 64 * 3 + 128 * 5 and d["write_bytes"] == 64 * 3 + 32 * 1
    assert d["moved_over_alg"] == (896 + 224) / 900.0
    out = tmp_path / "c.txt"
    subprocess.run([sys.executable, "-m", "recurrent_vision_backbone_chunkwise_amd.profiling", "counters",
                    "--pmc", str(tmp_path / "p1"), str(tmp_path / "p2"), str(tmp_path / "p3"), "--workload", "wl",
                    "--commands", f"rocprofv3 --pmc X -- python3 {ROOT}/bench.py", "--alg", "gla_seg_out=900",
                    "--out", str(out)], check=True, capture_output=True, cwd=ROOT)
    text = out.read_text()
    assert "$REPO/bench.py" in text and "gla_seg_out" in text and source_digest() in text


def test_digest_ignores_comments_and_layout():
    from recurrent_vision_backbone_chunkwise_amd.build import code_tokens
    a = 'int a = 1; // note\n/* block\n comment */ const char *s = "x // y /* z */";\nchar q = \'"\';   int b;\n'
    b = 'int a = 1;\nconst char *s = "x // y /* z */"; char q = \'"\'; int b; // other note\n'
    assert code_tokens(a) == code_tokens(b)
    assert code_tokens(a) != code_tokens(b.replace("int b", "int c"))
    assert '"x // y /* z */"' in code_tokens(a)


def test_counter_roles_for_a_kernel_that_alternates(tmp_path):
    """A library GEMM serving two projections in turn is split by dispatch order."""
    gemm = "Cijk_Ailk_Bljk_HHS_BH_MT256x256x64_MI16x16x1"
    write_multi(tmp_path / "p1", [(1, gemm, "SQ_INSTS_VALU_MFMA_MOPS_F16", 100), (2, gemm, "SQ_INSTS_VALU_MFMA_MOPS_F16", 40),
                                  (3, gemm, "SQ_INSTS_VALU_MFMA_MOPS_F16", 110), (4, gemm, "SQ_INSTS_VALU_MFMA_MOPS_F16", 50)])
    rows = profiling.counter_rows([str(tmp_path / "p1")], {"rocBLAS GEMM MT256x256x64": 2})
    assert rows["rocBLAS GEMM MT256x256x64#0"]["SQ_INSTS_VALU_MFMA_MOPS_F16"][0] == 105
    assert rows["rocBLAS GEMM MT256x256x64#1"]["SQ_INSTS_VALU_MFMA_MOPS_F16"][0] == 45
