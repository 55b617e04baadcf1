"""Build the gfx950 Muon library in-tree: ``python -m muon_newton_schulz_03_amd.build``.

Compiles every HIP source under ``csrc/`` into ``libmuon_mi355x.so`` next to
this file with hipcc.  Packed-fp32 instructions are disabled for the device
code (``-packed-fp32-ops``), as required on this platform; hipcc's host pass
warns that it does not know the feature, which is harmless.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB_NAME = "libmuon_mi355x.so"
LIB_PATH = os.path.join(HERE, LIB_NAME)
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc"), shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (set ROCM_PATH)")


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def build_library(verbose: bool = False, extra_flags=()) -> str:
    """Compile the shared library; returns its path.  Raises on compiler errors."""
    tmp = LIB_PATH + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-Wno-unused-command-line-argument",
           "-I", os.path.join(os.path.dirname(HERE), "include"),
           *extra_flags, *sources(), "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed with exit code {res.returncode}")
    if verbose and res.stderr.strip():
        # the host pass's note about the packed-fp32 feature is expected
        lines = [l for l in res.stderr.splitlines() if "packed-fp32-ops" not in l]
        if lines:
            sys.stderr.write("\n".join(lines) + "\n")
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build_library(verbose=True))
