"""Benchmark of the MI355X Muon step on the GPT-2 small hidden-matrix set.

One step = the whole hot path over all 72 hidden matrices of the 12-layer,
width-768 GPT-2 small model (overview page "The NanoGPT speedrun",
paragraph "Context"): momentum + Nesterov + Frobenius norm, T = 5 quintic
Newton-Schulz iterations, weight update, on fresh seeded bf16 gradients each
step (already resident in HBM; the plan is handed each step's gradient
buffers).  Prints one JSON line.

    python bench.py [--gpus 1] [--steps 50] [--warmup 5] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0
WORKLOAD = "gpt2_small"
PROFILES = os.path.join(ROOT, "profiles")


def kernel_source_hash() -> str:
    from muon_newton_schulz_03_amd.rocprof_summary import kernel_source_hash as h

    return h()


def work_model(shapes, T):
    """Algorithmic FLOPs of one iteration per product kind, and of a whole step (distinct
    entries of the symmetric products)."""
    gram = poly = upd = 0
    for r, c in shapes:
        m, n = min(r, c), max(r, c)
        gram += m * (m + 1) * n
        poly += m * m * (m + 1)
        upd += 2 * m * m * n
    dense = sum(T * (4 * min(r, c) ** 2 * max(r, c) + 2 * min(r, c) ** 3) for r, c in shapes)
    return {"gram": gram, "poly": poly, "update": upd, "step": T * (gram + poly + upd), "dense_step": dense}


def momentum_bytes(shapes, master: bool):
    """Algorithmic HBM bytes of the momentum kernel: G (bf16) + M read/write + X0 (bf16 [+ its low byte])."""
    p = sum(r * c for r, c in shapes)
    return p * (2 + 4 + 4 + 2 + (1 if master else 0))


def read_profile_value(summary: str, key: str):
    """One value of a committed rocprofv3 counter summary (profiles/); None when
    there is none or the kernels changed since the counters were taken."""
    path = os.path.join(PROFILES, f"{WORKLOAD}_{summary}.txt")
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as f:
        for line in f:
            if "=" in line and not line.startswith("#"):
                k, v = (s.strip() for s in line.split("=", 1))
                vals[k] = v
    if vals.get("kernel_source_hash") != kernel_source_hash():
        return None
    try:
        return float(vals[key])
    except (KeyError, ValueError):
        return None


def read_traffic(kind: str):
    """HBM bytes per launch of one kernel kind (FETCH_SIZE + WRITE_SIZE, calibrated)."""
    return read_profile_value("hbm_traffic", f"{kind}_hbm_bytes_per_launch")


def cpu_baseline(wl, budget_s: float = 12.0):
    """Time the fp64 oracle (as it stands) on a bounded sample: layer 0's six matrices, one step each."""
    import numpy as np
    import torch

    from muon_newton_schulz_03_amd import inputs
    from oracle import muon_oracle as O

    try:
        from threadpoolctl import threadpool_info
        threads = max((p.get("num_threads", 1) for p in threadpool_info()), default=os.cpu_count())
    except Exception:  # pragma: no cover
        threads = os.cpu_count()
    idx = list(range(6))
    grads = inputs.gradients(WORKLOAD, 0, indices=idx)
    zeros = [np.zeros(wl.shapes[i]) for i in idx]
    mz = [np.zeros(wl.shapes[i], np.float32) for i in idx]
    reps = 0
    t0 = time.perf_counter()
    while True:
        for k, i in enumerate(idx):
            O.muon_step(zeros[k], grads[k], mz[k], a=wl.coeffs[0], b=wl.coeffs[1], c=wl.coeffs[2], T=wl.T,
                        mu=wl.momentum, nesterov=wl.nesterov, lr=wl.lr)
        reps += 1
        el = time.perf_counter() - t0
        if el >= budget_s or reps >= 50:
            break
    layers = len(wl.shapes) // 6
    steps_per_s = reps / (el * layers)
    return {"value": steps_per_s, "unit": "steps/s", "cores": int(threads), "kind": "oracle",
            "sample": f"layer 0 (6 of 72 matrices: 4x768x768, 768x3072, 3072x768), {reps} oracle step(s) "
                      f"in {el:.1f} s, scaled by 12 layers"}


def after_timed_region(args, plan, grads, total, kw, wl, W, M, work, dom):
    """Measurements after the timed region: the dominant kernel in a one-stream plan,
    a per-iteration coefficient schedule, and the step replayed from a HIP graph."""
    import torch

    from muon_newton_schulz_03_amd import MuonStep

    # Per-iteration coefficient schedule (muon_step_schedule): the speedrun
    # quintic for 3 iterations, then a convergent quintic.
    sched = [wl.coeffs] * 3 + [(15 / 8, -10 / 8, 3 / 8)] * 2
    sched_steps = 20
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    plan.step(grads=grads[0], schedule=sched, momentum=wl.momentum, nesterov=wl.nesterov, lr=wl.lr)
    torch.cuda.synchronize()
    ev0.record()
    for t in range(sched_steps):
        plan.step(grads=grads[t % total], schedule=sched, momentum=wl.momentum, nesterov=wl.nesterov, lr=wl.lr)
    ev1.record()
    torch.cuda.synchronize()
    sched_ms = ev0.elapsed_time(ev1) / sched_steps

    # The step captured once in a HIP graph and replayed (fixed gradient buffers,
    # as when a training loop writes its gradients in place), outside the timed region.
    gbuf = [g.clone() for g in grads[0]]
    plan.step(grads=gbuf, **kw)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        plan.step(**kw)
    torch.cuda.synchronize()
    graph_steps = 50
    graph.replay()
    torch.cuda.synchronize()
    ev0.record()
    for _ in range(graph_steps):
        graph.replay()
    ev1.record()
    torch.cuda.synchronize()
    graph_ms = ev0.elapsed_time(ev1) / graph_steps
    del graph

    # The same kernel without the overlap: a one-stream plan, outside the timed region.
    plan1 = MuonStep(W, grads[0], M, x_master_iters=args.x_master_iters, groups=1)
    for t in range(2):
        plan1.step(grads=grads[t], **kw)
    plan1.profile(True, kinds=[dom])
    plan1.read_profile()
    one_steps = 10
    for t in range(one_steps):
        plan1.step(grads=grads[t % total], **kw)
    torch.cuda.synchronize()
    p1_ms, p1_cnt = plan1.read_profile()[dom]
    plan1.close()
    one_ms = p1_ms / p1_cnt
    if dom == "momentum":
        one_ach = momentum_bytes(wl.shapes, True) / (p1_cnt / one_steps) / (one_ms * 1e-3) / 1e9
        one_peak = PEAK_HBM_GBS
    else:
        one_ach = wl.T * work[dom] / (p1_cnt / one_steps) / (one_ms * 1e-3) / 1e12
        one_peak = PEAK_BF16_TFLOPS
    roof_one = {"bound": "hbm" if dom == "momentum" else "mfma", "achieved": one_ach, "peak": one_peak,
                "unit": "GB/s" if dom == "momentum" else "TFLOP/s",
                "frac": one_ach / one_peak, "kernel": dom, "ms_per_launch": one_ms,
                "note": f"one-stream plan (groups=1), {one_steps} steps after the timed region"}

    return {
        "roofline_one_stream": roof_one,
        "schedule": {"coeffs": [list(t) for t in sched], "ms_per_step": sched_ms, "steps_per_s": 1000.0 / sched_ms,
                     "note": f"muon_step_schedule, {sched_steps} steps after the timed region"},
        "graph": {"ms_per_step": graph_ms, "steps_per_s": 1000.0 / graph_ms,
                  "note": f"one step captured in a HIP graph, {graph_steps} replays after the timed region"},
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the passes after the timed region (one-stream roofline, schedule, graph)")
    ap.add_argument("--x-master-iters", type=int, default=-1)
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="run one plain 256 MiB device copy first (counter calibration)")
    ap.add_argument("--calibrate-mfma", action="store_true",
                    help="run a bf16 8192^3 torch GEMM three times first (MFMA-counter reference)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: the Muon step here has no multi-GPU path "
              f"(--gpus {args.gpus} requested)", file=sys.stderr)
        sys.exit(2)

    import torch

    from muon_newton_schulz_03_amd import MuonStep, inputs

    wl = inputs.workload(WORKLOAD)
    dev = torch.device("cuda:0")
    n = len(wl.shapes)
    total = args.warmup + args.steps
    print(f"[bench] {WORKLOAD}: {n} matrices, {wl.params} params, {total} gradient sets", file=sys.stderr,
          flush=True)
    grads = [inputs.gradients(WORKLOAD, t, device=dev) for t in range(total)]
    W = inputs.weights(wl.shapes, seed=11, device=dev)
    M = [torch.zeros(s, dtype=torch.float32, device=dev) for s in wl.shapes]
    if args.calibrate_copy:
        src = torch.empty(256 << 20, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    if args.calibrate_mfma:
        # a library GEMM of known FLOPs: its MFMA-busy reading and its FLOP rate
        # at its own clock check the counter normalisation (outside the Muon path)
        ga = torch.randn(8192, 8192, device=dev, dtype=torch.bfloat16)
        gb = torch.randn(8192, 8192, device=dev, dtype=torch.bfloat16)
        for _ in range(3):
            gc = ga @ gb
        torch.cuda.synchronize()
        del ga, gb, gc
    plan = MuonStep(W, grads[0], M, x_master_iters=args.x_master_iters)
    kw = dict(a=wl.coeffs[0], b=wl.coeffs[1], c=wl.coeffs[2], T=wl.T, momentum=wl.momentum,
              nesterov=wl.nesterov, lr=wl.lr)
    for t in range(args.warmup):
        plan.step(grads=grads[t], **kw)
    torch.cuda.synchronize()

    # Every launch timed with HIP events, outside the timed region (each event
    # record costs the stream a few microseconds): per-kind table and the
    # dominant kernel.
    prof_steps = 5
    plan.profile(True)
    plan.read_profile()
    for t in range(prof_steps):
        plan.step(grads=grads[t % args.warmup if args.warmup else 0], **kw)
    torch.cuda.synchronize()
    prof_all = plan.read_profile()
    work = work_model(wl.shapes, wl.T)
    per_kind = {}
    for k, (ms, cnt) in prof_all.items():
        if not cnt:
            continue
        per_kind[k] = {"ms_per_launch": ms / cnt, "launches_per_step": cnt / prof_steps}
        if k in ("gram", "poly", "update"):
            per_kind[k]["tflops"] = wl.T * work[k] / (cnt / prof_steps) / (ms / cnt * 1e-3) / 1e12
    if "momentum" in per_kind:
        mk = per_kind["momentum"]
        mk["gbs"] = momentum_bytes(wl.shapes, True) / mk["launches_per_step"] / (mk["ms_per_launch"] * 1e-3) / 1e9
    dom = max(("gram", "poly", "update", "momentum"), key=lambda k: prof_all[k][0])

    # timed region: K steps; HIP events (recorded by the library on this stream)
    # time the dominant kernel's launches only
    plan.profile(True, kinds=[dom])
    plan.read_profile()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for t in range(args.warmup, total):
        plan.step(grads=grads[t], **kw)
    stop.record()
    torch.cuda.synchronize()
    ms_total = start.elapsed_time(stop)
    prof = plan.read_profile()
    plan.profile(False)

    extras = {}
    if not args.no_extras:
        extras = after_timed_region(args, plan, grads, total, kw, wl, W, M, work, dom)
    plan.close()
    ms_step = ms_total / args.steps
    steps_per_s = 1000.0 / ms_step
    tflops = work["step"] * steps_per_s / 1e12
    d_ms, d_cnt = prof[dom]
    d_launch_ms = d_ms / d_cnt
    if dom == "momentum":
        achieved = momentum_bytes(wl.shapes, True) / (d_cnt / args.steps) / (d_launch_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": achieved / PEAK_HBM_GBS}
    else:
        achieved = wl.T * work[dom] / (d_cnt / args.steps) / (d_launch_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": achieved, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": achieved / PEAK_BF16_TFLOPS}
    roof["kernel"] = dom
    roof["ms_per_launch"] = d_launch_ms
    roof["launches_per_step"] = d_cnt / args.steps
    roof["traffic"] = read_traffic(dom)
    # share of SIMD cycles with the MFMA unit busy (rocprofv3 counters), when fresh
    roof["mfma_busy"] = read_profile_value("mfma_busy", f"{dom}_mfma_busy")
    roof["note"] = ("the plan runs two matrix groups on two streams, so each launch covers half the set "
                    "and shares the GPU with the other group's launches")

    out = {
        "metric": "Muon steps/s on GPT-2-small hidden set (T=5); % bf16 MFMA peak",
        "value": steps_per_s,
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "gpt2_small_hidden_72", "matrices": n, "params": wl.params, "T": wl.T,
                   "grad_dtype": "bf16", "weight_dtype": "f32", "momentum": wl.momentum, "nesterov": True,
                   "lr": wl.lr, "coeffs": list(wl.coeffs)},
        "tflops_algorithmic": tflops,
        "frac_bf16_peak": tflops / PEAK_BF16_TFLOPS,
        "tflops_dense_model": work["dense_step"] * steps_per_s / 1e12,
        "matrices_per_s": n * steps_per_s,
        "kernels": per_kind,
        "kernels_pass": f"{prof_steps} steps after warm-up with every launch timed, outside the timed region",
        "roofline": roof,
        **extras,
    }
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle baseline", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(wl)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
