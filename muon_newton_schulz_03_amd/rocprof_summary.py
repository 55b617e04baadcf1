"""Summaries of rocprofv3 output for the Muon kernels (text files for ``profiles/``).

Two summaries:

* kernel statistics from ``rocprofv3 --kernel-trace --stats --output-format csv``
  (``*_kernel_stats.csv`` and ``*_kernel_trace.csv``): per-kernel calls and
  average durations over the whole run; the mean duration per kind over the
  dispatches of bench.py's timed region (its last ``--steps`` steps; a step
  starts with the momentum pass of each matrix group, each followed by its
  norm or apply dispatch), beside what bench.py's own HIP
  events gave for its timed kernel in the same run (read from its JSON line
  in ``bench_log``, when given); the per-dispatch durations of the last step;
* HBM traffic from two ``--pmc`` runs (``FETCH_SIZE``, then ``WRITE_SIZE``,
  KiB per dispatch) of ``bench.py --calibrate-copy``, scaled by what the same
  counters read for the plain copy kernel of known size that run contains;
* MFMA busy from one ``--pmc SQ_VALU_MFMA_BUSY_CYCLES GRBM_GUI_ACTIVE`` run of
  ``bench.py --calibrate-mfma``: busy = SQ_VALU_MFMA_BUSY_CYCLES / (1024 SIMDs
  x GRBM_GUI_ACTIVE / 8 XCDs), i.e. the share of SIMD cycles whose MFMA unit
  is busy (the first counter sums over all SIMDs, the second over the XCDs).
  The run's library GEMM (bf16 8192^3) checks both sums: its busy cycles x
  1024 FLOP must equal its known FLOPs, and the clock GRBM_GUI_ACTIVE / 8 /
  dispatch time must stay within the chip's 2.4 GHz.

    python -m muon_newton_schulz_03_amd.rocprof_summary stats  <trace_dir> <out.txt> "<command>" [bench_log]
    python -m muon_newton_schulz_03_amd.rocprof_summary traffic <fetch_dir> <write_dir> <out.txt> "<commands>"
    python -m muon_newton_schulz_03_amd.rocprof_summary mfma    <pmc_dir> <out.txt> "<command>"
"""
from __future__ import annotations

import csv
import glob
import hashlib
import json
import os
import sys
from collections import defaultdict

HERE = os.path.dirname(os.path.abspath(__file__))
# the kernels and the launch structure (api.hip decides which launches a step makes)
KERNEL_SOURCES = [os.path.join(HERE, "csrc", f) for f in ("kernels.hip", "products.hip", "device_common.h", "muon_internal.h", "api.hip")]
COPY_BYTES = 256 << 20  # bench.py --calibrate-copy: one plain copy of 256 MiB

KINDS = {
    "momentum_kernel": "momentum",
    "norm_kernel": "norm",
    "ns_bf16_kernel<1": "gram",
    "ns_bf16_kernel<2": "poly",
    "ns_bf16_kernel<3": "update",
    "ns_stage_kernel<1": "gram",
    "ns_stage_kernel<2": "poly",
    "ns_stage_kernel<3": "update",
    "apply_kernel": "apply",
    "ns_fused_kernel": "fused",
}


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def kind_of(name: str):
    for key, kind in KINDS.items():
        if key in name:
            return kind
    return None


def _one(pattern: str) -> str:
    hits = glob.glob(pattern, recursive=True)
    if not hits:
        raise FileNotFoundError(pattern)
    return hits[0]


def _timed_steps(command: str) -> int:
    words = command.split()
    return int(words[words.index("--steps") + 1]) if "--steps" in words else 0


def _bench_line(bench_log: str):
    with open(bench_log) as f:
        for line in f:
            if line.startswith("{"):
                return json.loads(line)
    return None


def stats_summary(trace_dir: str, command: str, bench_log: str | None = None) -> str:
    stats = list(csv.DictReader(open(_one(os.path.join(trace_dir, "**", "*kernel_stats.csv")))))
    trace = list(csv.DictReader(open(_one(os.path.join(trace_dir, "**", "*kernel_trace.csv")))))
    lines = ["# rocprofv3 kernel statistics, Muon step on the GPT-2 small hidden set (72 matrices, T = 5)",
             f"# command: {command}",
             f"# kernel source hash: {kernel_source_hash()}",
             "# kind        calls   avg_us    min_us    max_us   kernel"]
    agg = defaultdict(lambda: [0, 0.0, float("inf"), 0.0, ""])
    for r in stats:
        k = kind_of(r["Name"])
        if not k:
            continue
        a = agg[(k, r["Name"])]
        calls = int(r["Calls"])
        a[0] += calls
        a[1] += float(r["TotalDurationNs"]) / 1000.0
        a[2] = min(a[2], float(r["MinNs"]) / 1000.0)
        a[3] = max(a[3], float(r["MaxNs"]) / 1000.0)
        a[4] = r["Name"]
    for (k, name), (calls, tot, mn, mx, _) in sorted(agg.items()):
        lines.append(f"{k:10s} {calls:7d} {tot / calls:9.1f} {mn:9.1f} {mx:9.1f}   {name[:70]}")
    mu = [r for r in trace if kind_of(r["Kernel_Name"])]
    mu.sort(key=lambda r: int(r["Dispatch_Id"]) if "Dispatch_Id" in r else 0)
    # step starts: a momentum dispatch not preceded by another group's momentum
    # pass (momentum, then norm or apply)
    head = ("momentum", "norm", "apply")
    starts = [i for i, r in enumerate(mu)
              if kind_of(r["Kernel_Name"]) == "momentum" and (i == 0 or kind_of(mu[i - 1]["Kernel_Name"]) not in head)]
    steps = _timed_steps(command)
    if steps:
        region = mu[starts[-steps]:] if len(starts) >= steps else []
        per = defaultdict(list)
        for r in region:
            per[kind_of(r["Kernel_Name"])].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1000.0)
        lines.append(f"# timed region: the last {steps} steps of the run; kind, dispatches, mean_us")
        for k in sorted(per):
            lines.append(f"timed_{k:10s} {len(per[k]):5d} {sum(per[k]) / len(per[k]):9.1f}")
    if bench_log:
        d = _bench_line(bench_log)
        if d and "roofline" in d:
            r = d["roofline"]
            lines.append(f"# bench.py in the same run, HIP events on its timed kernel ({r['kernel']}): "
                         f"{1000.0 * r['ms_per_launch']:.1f} us per launch, {d['ms_per_step']:.4f} ms per step")
    lines.append("# per-dispatch durations (us) of the last step, in launch order")
    for r in mu[starts[-1]:] if starts else []:
        dur = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1000.0
        lines.append(f"  {kind_of(r['Kernel_Name']):10s} {dur:9.1f}   {r['Kernel_Name'][:70]}")
    return "\n".join(lines) + "\n"


def _counter_rows(pmc_dir: str, counter: str):
    rows = list(csv.DictReader(open(_one(os.path.join(pmc_dir, "**", "*counter_collection.csv")))))
    return [r for r in rows if r["Counter_Name"] == counter]


def traffic_summary(fetch_dir: str, write_dir: str, command: str) -> str:
    out = []
    scale = {}
    per_kind = {}
    for counter, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        rows = _counter_rows(d, counter)
        copies = [float(r["Counter_Value"]) for r in rows
                  if "copy" in r["Kernel_Name"].lower() and int(r["Grid_Size"]) > 0]
        # the calibration copy is the largest copy kernel of the run
        kib = max(copies) if copies else None
        scale[counter] = COPY_BYTES / (kib * 1024.0) if kib else None
        acc = defaultdict(list)
        for r in rows:
            k = kind_of(r["Kernel_Name"])
            if k:
                acc[k].append(float(r["Counter_Value"]) * 1024.0)
        per_kind[counter] = acc
    out.append("# HBM traffic per dispatch from rocprofv3 counters (FETCH_SIZE, WRITE_SIZE; KiB per dispatch)")
    out.append(f"# commands: {command}")
    out.append("# scale = known bytes of a plain 256 MiB copy / bytes the counter reports for it")
    out.append(f"fetch_scale = {scale['FETCH_SIZE']}")
    out.append(f"write_scale = {scale['WRITE_SIZE']}")
    out.append(f"kernel_source_hash = {kernel_source_hash()}")
    for k in ("momentum", "gram", "poly", "update"):
        f = per_kind["FETCH_SIZE"].get(k, [])
        w = per_kind["WRITE_SIZE"].get(k, [])
        if not f or not w:
            continue
        fs = scale["FETCH_SIZE"] or 1.0
        ws = scale["WRITE_SIZE"] or 1.0
        fb = sum(f) / len(f) * fs
        wb = sum(w) / len(w) * ws
        out.append(f"{k}_fetch_bytes_per_launch = {fb:.0f}")
        out.append(f"{k}_write_bytes_per_launch = {wb:.0f}")
        out.append(f"{k}_hbm_bytes_per_launch = {fb + wb:.0f}")
    return "\n".join(out) + "\n"


N_XCD = 8          # MI355X: XCDs (GRBM_GUI_ACTIVE sums over them)
N_SIMD = 256 * 4   # MI355X: CUs x SIMDs (SQ_VALU_MFMA_BUSY_CYCLES sums over them)
GEMM_FLOPS = 2.0 * 8192 ** 3
PEAK_BF16_PER_CLOCK = 256 * 4096.0  # dense bf16 FLOP per clock (2.5 PFLOP/s at 2.4 GHz)


def mfma_summary(pmc_dir: str, command: str) -> str:
    rows = list(csv.DictReader(open(_one(os.path.join(pmc_dir, "**", "*counter_collection.csv")))))
    disp = defaultdict(dict)
    for r in rows:
        d = disp[r["Dispatch_Id"]]
        d["name"] = r["Kernel_Name"]
        d["ns"] = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
        d[r["Counter_Name"]] = float(r["Counter_Value"])
    per_kind = defaultdict(list)
    gemm = []
    for d in disp.values():
        if "SQ_VALU_MFMA_BUSY_CYCLES" not in d or "GRBM_GUI_ACTIVE" not in d or d["GRBM_GUI_ACTIVE"] <= 0:
            continue
        busy = d["SQ_VALU_MFMA_BUSY_CYCLES"] / (N_SIMD * d["GRBM_GUI_ACTIVE"] / N_XCD)
        clock = d["GRBM_GUI_ACTIVE"] / N_XCD / d["ns"]  # GHz
        k = kind_of(d["name"])
        if k:
            per_kind[k].append((busy, clock))
        elif busy > 0.2 and d["ns"] > 200_000:  # the calibration GEMM (the only other MFMA kernel)
            # one busy SIMD cycle of a bf16 32x32x16 / 16x16x32 MFMA is 1024 FLOP
            gemm.append((busy, clock, d["SQ_VALU_MFMA_BUSY_CYCLES"] * 1024.0 / GEMM_FLOPS))
    out = ["# MFMA busy per dispatch from rocprofv3 counters (SQ_VALU_MFMA_BUSY_CYCLES, GRBM_GUI_ACTIVE)",
           f"# command: {command}",
           f"# busy = SQ_VALU_MFMA_BUSY_CYCLES / ({N_SIMD} SIMDs x GRBM_GUI_ACTIVE / {N_XCD} XCDs), mean over"
           " dispatches; the timer window of a short dispatch includes a few idle microseconds, so short"
           " kernels read slightly low",
           f"kernel_source_hash = {kernel_source_hash()}"]
    for k in ("momentum", "gram", "poly", "update"):
        v = per_kind.get(k)
        if not v:
            continue
        out.append(f"{k}_mfma_busy = {sum(b for b, _ in v) / len(v):.4f}")
    if gemm:
        out.append("# reference: library bf16 GEMM 8192^3.  Its busy SIMD cycles x 1024 FLOP should equal its")
        out.append("# 2 * 8192^3 FLOP (ratio 1: the counter sums over SIMDs), and the clock GRBM_GUI_ACTIVE / 8 /")
        out.append("# dispatch time of this long dispatch should stay within the 2.4 GHz maximum (the timer sums over XCDs).")
        out.append(f"gemm_mfma_busy = {sum(g[0] for g in gemm) / len(gemm):.4f}")
        out.append(f"gemm_clock_ghz = {sum(g[1] for g in gemm) / len(gemm):.3f}")
        out.append(f"gemm_counted_over_known_flops = {sum(g[2] for g in gemm) / len(gemm):.4f}")
    return "\n".join(out) + "\n"


def main(argv):
    if argv[0] == "stats":
        text = stats_summary(argv[1], argv[3], argv[4] if len(argv) > 4 else None)
        out = argv[2]
    elif argv[0] == "traffic":
        text = traffic_summary(argv[1], argv[2], argv[4])
        out = argv[3]
    elif argv[0] == "mfma":
        text = mfma_summary(argv[1], argv[3])
        out = argv[2]
    else:
        raise SystemExit(__doc__)
    with open(out, "w") as f:
        f.write(text)
    print(text)


if __name__ == "__main__":
    main(sys.argv[1:])
