"""The rocprofv3 summary tool and bench.py's reading of its output, on synthetic CSV files.

The values are chosen so that every expected figure follows by hand from the
definitions in the tool's docstring: the copy calibration (known bytes / counted
bytes), the per-dispatch MFMA busy share (busy cycles over 1024 SIMDs times the
per-XCD clock count) and the kernel-statistics aggregation.
"""
import csv
import os

import pytest

import bench
from muon_newton_schulz_03_amd import rocprof_summary as R


def write_csv(path, header, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(header)
        w.writerows(rows)


def counters(path, counter, rows):
    # rows: (kernel name, grid size, KiB per dispatch)
    write_csv(path, ["Dispatch_Id", "Kernel_Name", "Grid_Size", "Counter_Name", "Counter_Value"],
              [(i, name, grid, counter, kib) for i, (name, grid, kib) in enumerate(rows)])


def values(text):
    out = {}
    for line in text.splitlines():
        if "=" in line and not line.startswith("#"):
            k, v = (s.strip() for s in line.split("=", 1))
            out[k] = v
    return out


def test_traffic_is_scaled_by_the_copy_calibration(tmp_path):
    copy_kib = R.COPY_BYTES / 1024
    upd = "void muon::ns_stage_kernel<3, false, 5>(muon::StageArgs)"
    # FETCH_SIZE reads half the copy's bytes (scale 2), WRITE_SIZE all of them (scale 1)
    counters(str(tmp_path / "f" / "run_counter_collection.csv"), "FETCH_SIZE",
             [("__amd_rocclr_copyBuffer", 4096, copy_kib / 2), ("__amd_rocclr_copyBuffer", 0, 1.0),
              (upd, 512, 100.0), (upd, 512, 300.0), ("other_kernel", 64, 7.0)])
    counters(str(tmp_path / "w" / "run_counter_collection.csv"), "WRITE_SIZE",
             [("__amd_rocclr_copyBuffer", 4096, copy_kib), (upd, 512, 50.0), (upd, 512, 150.0)])
    v = values(R.traffic_summary(str(tmp_path / "f"), str(tmp_path / "w"), "cmd"))
    assert float(v["fetch_scale"]) == pytest.approx(2.0)
    assert float(v["write_scale"]) == pytest.approx(1.0)
    # mean KiB per dispatch x 1024 x scale
    assert float(v["update_fetch_bytes_per_launch"]) == pytest.approx(200.0 * 1024 * 2)
    assert float(v["update_write_bytes_per_launch"]) == pytest.approx(100.0 * 1024)
    assert float(v["update_hbm_bytes_per_launch"]) == pytest.approx(200.0 * 1024 * 2 + 100.0 * 1024)
    assert "gram_fetch_bytes_per_launch" not in v
    assert v["kernel_source_hash"] == R.kernel_source_hash()


def test_mfma_busy_normalisation(tmp_path):
    rows = []
    ns = 1_000_000  # 1 ms dispatches
    active = 8 * 1.8e6  # GRBM_GUI_ACTIVE sums 8 XCDs: 1.8e6 clocks each, 1.8 GHz over 1 ms
    gemm_flops = 2.0 * 8192 ** 3
    dispatches = [
        ("void muon::ns_stage_kernel<1, false, 0>(muon::StageArgs)", 0.25 * 1024 * active / 8),
        ("void muon::ns_stage_kernel<1, false, 0>(muon::StageArgs)", 0.35 * 1024 * active / 8),
        ("Cijk_gemm_bf16", gemm_flops / 1024),
    ]
    for i, (name, busy) in enumerate(dispatches):
        for counter, value in (("SQ_VALU_MFMA_BUSY_CYCLES", busy), ("GRBM_GUI_ACTIVE", active)):
            rows.append((i, name, 0, ns, counter, value))
    write_csv(str(tmp_path / "m" / "run_counter_collection.csv"),
              ["Dispatch_Id", "Kernel_Name", "Start_Timestamp", "End_Timestamp", "Counter_Name", "Counter_Value"],
              rows)
    v = values(R.mfma_summary(str(tmp_path / "m"), "cmd"))
    assert float(v["gram_mfma_busy"]) == pytest.approx(0.30, abs=1e-4)
    assert float(v["gemm_clock_ghz"]) == pytest.approx(1.8, abs=1e-3)
    assert float(v["gemm_counted_over_known_flops"]) == pytest.approx(1.0, abs=1e-4)
    assert float(v["gemm_mfma_busy"]) == pytest.approx(gemm_flops / 1024 / (1024 * active / 8), abs=1e-4)


def test_kernel_statistics(tmp_path):
    gram = "void muon::ns_stage_kernel<1, false, 0>(muon::StageArgs)"
    mom = "muon::momentum_kernel(muon::MomArgs)"
    write_csv(str(tmp_path / "s" / "run_kernel_stats.csv"), ["Name", "Calls", "TotalDurationNs", "MinNs", "MaxNs"],
              [(gram, 4, 400_000, 90_000, 110_000), (mom, 2, 300_000, 140_000, 160_000), ("torch_kernel", 9, 9, 1, 1)])
    write_csv(str(tmp_path / "s" / "run_kernel_trace.csv"), ["Kernel_Name", "Start_Timestamp", "End_Timestamp"],
              [(mom, 0, 150_000), (gram, 160_000, 260_000), (gram, 270_000, 370_000)])
    text = R.stats_summary(str(tmp_path / "s"), "cmd")
    head = text.split("# per-dispatch durations")[0]
    lines = {ln.split()[0]: ln.split() for ln in head.splitlines() if ln and not ln.startswith("#")}
    assert lines["gram"][1:5] == ["4", "100.0", "90.0", "110.0"]
    assert lines["momentum"][1:5] == ["2", "150.0", "140.0", "160.0"]
    assert "torch_kernel" not in text
    # the last step starts at its momentum dispatch
    tail = text.split("in launch order\n")[1].split()
    assert tail[:2] == ["momentum", "150.0"] and tail.count("gram") == 2


def test_bench_reads_values_only_for_the_current_sources(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    path = tmp_path / f"{bench.WORKLOAD}_hbm_traffic.txt"
    assert bench.read_traffic("update") is None  # no summary
    path.write_text(f"# x\nkernel_source_hash = {R.kernel_source_hash()}\nupdate_hbm_bytes_per_launch = 123\n")
    assert bench.read_traffic("update") == 123.0
    assert bench.read_traffic("gram") is None  # no such line
    path.write_text("kernel_source_hash = 0000000000000000\nupdate_hbm_bytes_per_launch = 123\n")
    assert bench.read_traffic("update") is None  # kernels changed since the counters were taken


def test_timed_region_means_and_bench_figure(tmp_path):
    """Two matrix groups: a step opens with (momentum, norm) per group; the timed
    region is the last --steps steps, and its per-kind means use those
    dispatches only."""
    names = {"mom": "muon::momentum_kernel(muon::MomArgs)", "norm": "muon::norm_kernel(muon::DevMat const*)",
             "gram": "void muon::ns_stage_kernel<1, false, 0>(muon::StageArgs)",
             "upd": "void muon::ns_stage_kernel<3, false, 5>(muon::StageArgs)"}
    rows, t, did = [], 0, 0

    def step(gram_us, upd_us):
        nonlocal t, did
        for k, us in (("mom", 100), ("norm", 5), ("mom", 100), ("norm", 5),
                      ("gram", gram_us), ("gram", gram_us), ("upd", upd_us), ("upd", upd_us + 20)):
            did += 1
            rows.append((did, names[k], t, t + us * 1000))
            t += us * 1000 + 1000
    step(500, 900)  # a warm-up step: slow, outside the timed region
    step(90, 150)
    step(110, 170)
    write_csv(str(tmp_path / "s" / "run_kernel_trace.csv"), ["Dispatch_Id", "Kernel_Name", "Start_Timestamp", "End_Timestamp"],
              list(reversed(rows)))  # file order does not matter: dispatches are sorted by id
    write_csv(str(tmp_path / "s" / "run_kernel_stats.csv"), ["Name", "Calls", "TotalDurationNs", "MinNs", "MaxNs"],
              [(names["gram"], 6, 1, 1, 1)])
    log = tmp_path / "bench.log"
    log.write_text('[bench] text\n{"ms_per_step": 1.5, "roofline": {"kernel": "update", "ms_per_launch": 0.171}}\n')
    text = R.stats_summary(str(tmp_path / "s"), "rocprofv3 -- python bench.py --steps 2 --warmup 1", str(log))
    timed = {ln.split()[0]: ln.split()[1:] for ln in text.splitlines() if ln.startswith("timed_")}
    assert timed["timed_gram"] == ["4", "100.0"]
    assert timed["timed_update"] == ["4", "170.0"]  # (150 + 170 + 170 + 190) / 4
    assert timed["timed_momentum"] == ["4", "100.0"]
    assert "update): 171.0 us per launch, 1.5000 ms per step" in text
    # the last step, from the first group's momentum pass on
    tail = text.split("in launch order\n")[1].split("\n")
    assert [ln.split()[0] for ln in tail if ln] == ["momentum", "norm", "momentum", "norm", "gram", "gram", "update", "update"]
