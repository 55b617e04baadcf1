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
