"""bench.py's host-side pieces: the one-GPU guard, the work model, the profile summaries."""
import os
import subprocess
import sys

import bench
from muon_newton_schulz_03_amd import inputs
from oracle import muon_oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_multi_gpu_request_exits_with_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode != 0 and "one GPU" in r.stderr


def test_work_model_matches_oracle_counts():
    wl = inputs.workload("gpt2_small")
    w = bench.work_model(wl.shapes, wl.T)
    assert w["step"] == sum(O.ns_flops_algorithmic(r, c, wl.T) for r, c in wl.shapes)
    assert w["dense_step"] == sum(O.ns_flops_dense(r, c, wl.T) for r, c in wl.shapes)
    assert abs(w["step"] - 1.1422e12) / 1.1422e12 < 1e-3
    assert w["update"] == 130_459_631_616  # 48 * 2 * 768^3 + 24 * 2 * 768^2 * 3072
    assert bench.momentum_bytes(wl.shapes, True) == wl.params * 13


def test_profile_summaries_are_text_with_commands():
    prof = os.path.join(ROOT, "profiles")
    for name in os.listdir(prof):
        path = os.path.join(prof, name)
        assert name.endswith((".txt", ".md")), name
        text = open(path).read()
        assert "rocprofv3" in text and len(text) < 20000


def test_cpu_info_names_the_host():
    nproc, model, blas = bench.cpu_info()
    assert nproc >= 1 and isinstance(model, str) and model
    assert blas is None or blas >= 1


def test_traffic_model_counts_each_buffer_once():
    wl = inputs.workload("gpt2_small")
    t = bench.traffic_model(wl.shapes, wl.T, kmaster=3)
    mn = sum(r * c for r, c in wl.shapes)            # X elements of the set
    mm = sum(min(r, c) ** 2 for r, c in wl.shapes)   # A (and B) elements of the set
    assert (mn, mm) == (84_934_656, 42_467_328)
    assert t["momentum"] == 13 * mn
    assert t["gram_per_iter"] == 2 * mn + 2 * mm and t["poly_per_iter"] == 4 * mm
    base = 2 * mm + 2 * mn                           # B and X read by every update
    assert t["update_per_iter"] == [base + mn + 3 * mn, base + mn + 3 * mn, base + mn + 2 * mn, base + 2 * mn,
                                    base + 8 * mn]
    assert t["update"] == sum(t["update_per_iter"]) and t["gram"] == 5 * t["gram_per_iter"]
    assert bench.traffic_model(wl.shapes, wl.T, kmaster=0)["momentum"] == 12 * mn


def test_roofline_takes_the_roof_with_the_longer_floor():
    # 1 GFLOP in 0.4 us at the bf16 peak; 1 MB in 0.125 us at the HBM peak
    r = bench.kernel_roofline("k", 1e9, 1e6, 0.001)
    assert r["bound"] == "mfma" and abs(r["frac"] - 0.4) < 1e-9 and abs(r["hbm_view"]["frac"] - 0.125) < 1e-9
    r = bench.kernel_roofline("k", 1e9, 1e7, 0.002)
    assert r["bound"] == "hbm" and abs(r["frac"] - 0.625) < 1e-9 and abs(r["mfma_view"]["frac"] - 0.2) < 1e-9
    assert bench.kernel_roofline("m", 0, 8e6, 0.001)["frac"] == 1.0
    wl = inputs.workload("gpt2_small")
    w, t = bench.work_model(wl.shapes, wl.T), bench.traffic_model(wl.shapes, wl.T)
    # every launch of this set has a longer HBM floor than MFMA floor
    total = t["momentum"] + t["gram"] + t["poly"] + t["update"]
    assert abs(bench.step_floor_ms(w, t, wl.T) - total / 8e12 * 1e3) < 1e-9
