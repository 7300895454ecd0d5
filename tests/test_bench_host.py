"""Host logic of bench.py, on the CPU (no GPU call): the one-GPU contract, the profile
summarizers (calibrated traffic, MFMA utilization, wave-time counters) on synthetic rocprofv3
counter files, the source hash that ties committed profiles to the kernels they measured, and
the token counts of the extra workloads the default run measures."""
import csv
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import bench  # noqa: E402
import bit_ternary_weight_absmean_amd as bt  # noqa: E402

M_PREFILL = 2048
SHAPES_2B = [("qkv", 3840, 2560), ("o", 2560, 2560), ("gate_up", 13824, 2560), ("down", 2560, 6912)]


def run_bench(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                          cwd=ROOT, timeout=600)


def write_counters(d, rows):
    """A rocprofv3 counter_collection.csv with the columns the summarizers read."""
    os.makedirs(d, exist_ok=True)
    fields = ["Dispatch_Id", "Grid_Size", "Kernel_Name", "Counter_Name", "Counter_Value", "Start_Timestamp",
              "End_Timestamp"]
    with open(os.path.join(d, "run_counter_collection.csv"), "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=fields)
        w.writeheader()
        for r in rows:
            w.writerow({k: r.get(k, 0) for k in fields})
    return d


def gemm_grid(M, N, K):
    """Threads of the k_gemm launch the step's route makes (as the launcher sizes it)."""
    tiles = -(-M // 64) * -(-N // 256)
    full, splits = bt.gemm_split_plan(M, N, K)
    full = tiles if splits == 1 else full
    return 256 * 8 * (-(-full // 8) + -(-(tiles - full) // 8) * splits)


def test_more_than_one_gpu_is_refused():
    r = run_bench("--gpus", "2")
    assert r.returncode == 2
    assert "exactly one GPU" in r.stderr


def test_extra_workloads_are_parity_covered_token_counts():
    # every configuration the default run adds is run at a token count whose kernel instances
    # the plan-coverage test ties to a GPU parity case
    for name, m in bench.EXTRA_WORKLOADS:
        assert m in bench.WORKLOAD_M[name], (name, m)


def test_summarize_pmc_scales_by_the_copy_calibration(tmp_path):
    gemm = "void bt::(anonymous namespace)::k_gemm<64, 256, 1, 4, 3, 3, false>(...)"
    copy = "void at::native::elementwise_kernel<128, 4>(...)"
    f = write_counters(str(tmp_path / "f"), [{"Kernel_Name": gemm, "Counter_Name": "FETCH_SIZE", "Counter_Value": v}
                                            for v in (900.0, 1100.0)])
    w = write_counters(str(tmp_path / "w"), [{"Kernel_Name": gemm, "Counter_Name": "WRITE_SIZE", "Counter_Value": v}
                                            for v in (400.0, 600.0)])
    # a 1 GiB copy: FETCH_SIZE reads half the bytes (factor 2), WRITE_SIZE all of them (factor 1)
    cf = write_counters(str(tmp_path / "cf"), [{"Kernel_Name": copy, "Counter_Name": "FETCH_SIZE",
                                                "Counter_Value": (1 << 30) / 2 / 1024}])
    cw = write_counters(str(tmp_path / "cw"), [{"Kernel_Name": copy, "Counter_Name": "WRITE_SIZE",
                                                "Counter_Value": (1 << 30) / 1024}])
    out = tmp_path / "traffic.json"
    r = run_bench("--workload", "2b_prefill", "--m", str(M_PREFILL), "--summarize-pmc", f, w, cf, cw, str(out),
                  "--command", "synthetic")
    assert r.returncode == 0, r.stderr
    d = json.loads(out.read_text())
    assert d["kernel"] == "k_gemm"
    assert d["copy_calibration"]["fetch_factor"] == 2.0 and d["copy_calibration"]["write_factor"] == 1.0
    assert d["traffic_bytes_per_launch"] == round(1000.0 * 1024 * 2.0 + 500.0 * 1024 * 1.0)
    assert d["source_sha256"] == bench.source_hash("k_gemm")
    # the algorithmic bytes are the mean over the workload's four shapes
    alg = [bench.gemv_bytes(M_PREFILL, N, K) for _, N, K in SHAPES_2B]
    assert d["algorithmic_bytes_per_launch"] == round(sum(alg) / len(alg))


def test_summarize_mfma_counts_ops_per_shape(tmp_path):
    gemm = "void bt::(anonymous namespace)::k_gemm<64, 256, 1, 4, 3, 3, false>(...)"
    rows = []
    for i, (_, N, K) in enumerate(SHAPES_2B):
        ops = 2 * M_PREFILL * N * K
        common = {"Dispatch_Id": i, "Kernel_Name": gemm, "Start_Timestamp": 0, "End_Timestamp": 20_000}
        rows.append({**common, "Counter_Name": "MfmaUtil", "Counter_Value": 10.0 * (i + 1)})
        rows.append({**common, "Counter_Name": "SQ_INSTS_VALU_MFMA_MOPS_I8", "Counter_Value": ops / 512})
    d_in = write_counters(str(tmp_path / "m"), rows)
    out = tmp_path / "mfma.json"
    r = run_bench("--workload", "2b_prefill", "--m", str(M_PREFILL), "--summarize-mfma", d_in, str(out),
                  "--command", "synthetic")
    assert r.returncode == 0, r.stderr
    d = json.loads(out.read_text())
    assert d["int8_mfma_ops_per_launch"] == d["algorithmic_ops_per_launch"]
    assert d["mfma_util_percent_mean"] == 25.0
    assert {k.split()[0] for k in d["per_shape"]} == {n for n, _, _ in SHAPES_2B}
    # 20 us per dispatch: TOPS under counters = ops / 20 us
    q = d["per_shape"]["qkv 3840x2560"]
    assert q["TOPS_under_counters"] == round(2 * M_PREFILL * 3840 * 2560 / 20e-6 / 1e12, 1)


def test_summarize_sq_labels_shapes_by_launch_grid(tmp_path):
    gemm = "void bt::(anonymous namespace)::k_gemm<64, 256, 1, 4, 3, 3, false>(...)"
    per_wave = {"SQ_WAVE_CYCLES": 1000, "SQ_ACTIVE_INST_ANY": 400, "SQ_ACTIVE_INST_VALU": 300, "SQ_WAIT_ANY": 250,
                "SQ_WAIT_INST_ANY": 200, "SQ_LDS_BANK_CONFLICT": 3, "SQ_INSTS_LDS": 2}
    dirs = []
    for p, counters in enumerate(bench.SQ_PASSES):
        rows = []
        for i, (_, N, K) in enumerate(SHAPES_2B):
            grid = gemm_grid(M_PREFILL, N, K)
            waves = grid // 64
            for c in counters:
                v = waves if c == "SQ_WAVES" else per_wave.get(c, 1) * waves
                rows.append({"Dispatch_Id": i, "Grid_Size": grid, "Kernel_Name": gemm, "Counter_Name": c,
                             "Counter_Value": v})
        dirs.append(write_counters(str(tmp_path / f"sq{p}"), rows))
    out = tmp_path / "sq.md"
    r = run_bench("--workload", "2b_prefill", "--m", str(M_PREFILL), "--summarize-sq", dirs[0], dirs[1], str(out))
    assert r.returncode == 0, r.stderr
    table = [ln for ln in out.read_text().splitlines() if ln.startswith("| ") and "tiles" in ln]
    assert len(table) == 4
    for ln in table:
        cells = [c.strip() for c in ln.strip("|").split("|")]
        # wave-cycles per wave, issuing, VALU share of issue, at s_waitcnt, dependency stalls, conflicts
        assert cells[2:] == ["1000", "40%", "75%", "25%", "20%", "1.50"], ln
    assert any("down 2560x6912" in ln and "split in" in ln for ln in table)  # the tail-split route's grid


def test_source_hash_ignores_comments_and_blank_lines(tmp_path, monkeypatch):
    src = tmp_path / "k.hip"
    monkeypatch.setattr(bench, "CSRC", str(tmp_path))
    monkeypatch.setitem(bench.KERNEL_SOURCES, "k_test", ["k.hip"])
    src.write_text("int x = 1; // a comment\n\n/* a block */ int y;\n")
    h = bench.source_hash("k_test")
    src.write_text("  int x = 1;   // another comment\n/* a block\n   over lines */ int y;\n\n\n")
    assert bench.source_hash("k_test") == h
    src.write_text("int x = 2;\nint y;\n")
    assert bench.source_hash("k_test") != h


@pytest.mark.parametrize("kernel", sorted(bench.KERNEL_SOURCES))
def test_kernel_sources_exist(kernel):
    for f in bench.KERNEL_SOURCES[kernel]:
        assert os.path.exists(os.path.join(bench.CSRC, f)), f


def test_summarize_trace_takes_the_median_of_runs(tmp_path):
    """Several trace runs of one command: the dominant kernel's figure is the median of the runs' means."""
    dec = "void bt::(anonymous namespace)::k_linear_decode<1, 8, 2, 1, false>(...)"
    fields = ["Kernel_Name", "Grid_Size", "Workgroup_Size", "Start_Timestamp", "End_Timestamp"]
    dirs = []
    for run, dur_ns in enumerate((3000, 5000, 4000)):
        d = tmp_path / f"tr{run}"
        d.mkdir()
        with open(d / "run_kernel_trace.csv", "w", newline="") as fh:
            w = csv.DictWriter(fh, fieldnames=fields)
            w.writeheader()
            for i in range(10):  # dispatches 8 us apart
                t0 = 1_000_000 * run + 8000 * i
                w.writerow({"Kernel_Name": dec, "Grid_Size": 122880, "Workgroup_Size": 512, "Start_Timestamp": t0,
                            "End_Timestamp": t0 + dur_ns})
        dirs.append(str(d))
    out = tmp_path / "trace.md"
    r = run_bench("--summarize-trace", ",".join(dirs), str(out), "--command", "synthetic")
    assert r.returncode == 0, r.stderr
    rec = json.loads((tmp_path / "trace.json").read_text())
    assert rec["run_mean_duration_us"] == [3.0, 5.0, 4.0]
    assert rec["mean_duration_us"] == 4.0
    assert rec["dispatches"] == 30
    assert rec["mean_interval_us"] == 8.0
