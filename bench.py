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


def traffic_model(shapes, T, kmaster: int = 3, w_bytes: int = 4):
    """Algorithmic HBM bytes of one step per kernel kind, bf16 products (every
    short side >= 128), and of each update launch's iteration: what each kernel
    must read and write once, with operand re-reads across tiles served from L2.

    momentum: G (bf16) + M read and written + X0 (bf16 and, with kmaster > 0,
    its low byte).  Per iteration t: Gram reads X (bf16) and writes A (m x m,
    stored in full); the polynomial reads A and writes B; the update reads B and
    X, X's low bytes when t <= kmaster, and writes the new X (and its low bytes
    when t < kmaster), or, at t = T, reads and writes the fp32 weights instead.
    B's diagonal words (4 m bytes per matrix) are left out."""
    mom = gram = poly = 0
    upd = [0] * T
    for r, c in shapes:
        m, n = min(r, c), max(r, c)
        mn, mm = m * n, m * m
        mom += mn * (2 + 4 + 4 + 2 + (1 if kmaster > 0 else 0))
        gram += mn * 2 + mm * 2
        poly += mm * 2 + mm * 2
        for t in range(1, T + 1):
            b = mm * 2 + mn * 2 + (mn if t <= kmaster else 0)
            b += 2 * mn * w_bytes if t == T else mn * 2 + (mn if t < kmaster else 0)
            upd[t - 1] += b
    return {"momentum": mom, "gram": T * gram, "poly": T * poly, "update": sum(upd), "update_per_iter": upd,
            "gram_per_iter": gram, "poly_per_iter": poly}


def step_floor_ms(work, traffic, T):
    """The step's roofline floor: every launch at the larger of its MFMA time
    (algorithmic FLOPs at the bf16 peak) and its HBM time (algorithmic bytes at
    the HBM peak), summed over the step; momentum is HBM only.  The two matrix
    groups split FLOPs and bytes alike, so whole-set sums per iteration serve."""
    f = lambda flops, nbytes: max(flops / (PEAK_BF16_TFLOPS * 1e12), nbytes / (PEAK_HBM_GBS * 1e9))
    s = traffic["momentum"] / (PEAK_HBM_GBS * 1e9)
    for t in range(T):
        s += f(work["gram"], traffic["gram_per_iter"]) + f(work["poly"], traffic["poly_per_iter"])
        s += f(work["update"], traffic["update_per_iter"][t])
    return 1e3 * s


def kernel_roofline(kind, flops, nbytes, ms):
    """Roofline of one kernel from its algorithmic FLOPs and bytes per launch and
    its average launch time: bound is the roof with the longer floor; the other
    roof's view is kept beside it."""
    t_f = flops / (PEAK_BF16_TFLOPS * 1e12) if flops else 0.0
    t_b = nbytes / (PEAK_HBM_GBS * 1e9)
    hbm = {"achieved": nbytes / (ms * 1e-3) / 1e9, "peak": PEAK_HBM_GBS, "unit": "GB/s"}
    hbm["frac"] = hbm["achieved"] / PEAK_HBM_GBS
    if not flops:
        return {"bound": "hbm", **hbm}
    mfma = {"achieved": flops / (ms * 1e-3) / 1e12, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s"}
    mfma["frac"] = mfma["achieved"] / PEAK_BF16_TFLOPS
    floors = {"mfma_us": 1e6 * t_f, "hbm_us": 1e6 * t_b}
    if t_b > t_f:
        return {"bound": "hbm", **hbm, "floors_per_launch": floors, "mfma_view": mfma}
    return {"bound": "mfma", **mfma, "floors_per_launch": floors, "hbm_view": hbm}


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


def cpu_info():
    """Logical CPUs this process may use, the CPU model, and the BLAS thread count."""
    try:
        nproc = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        nproc = os.cpu_count()
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:  # pragma: no cover
        pass
    try:
        from threadpoolctl import threadpool_info
        blas = max((p.get("num_threads", 1) for p in threadpool_info() if p.get("user_api") == "blas"), default=None)
    except Exception:  # pragma: no cover
        blas = None
    return nproc, model, blas


def cpu_baseline(wl, reps: int = 3):
    """Time the fp64 oracle (as it stands) on full steps of the workload: all 72
    matrices, one Muon step each, `reps` times; the median step is the value."""
    import numpy as np

    from muon_newton_schulz_03_amd import inputs
    from oracle import muon_oracle as O

    nproc, model, blas = cpu_info()
    grads = inputs.gradients(WORKLOAD, 0)
    times = []
    for _ in range(reps):
        mz = [np.zeros(s, np.float32) for s in wl.shapes]
        t0 = time.perf_counter()
        for i, shape in enumerate(wl.shapes):
            O.muon_step(np.zeros(shape), grads[i], mz[i], a=wl.coeffs[0], b=wl.coeffs[1], c=wl.coeffs[2],
                        T=wl.T, mu=wl.momentum, nesterov=wl.nesterov, lr=wl.lr)
        times.append(time.perf_counter() - t0)
    med = float(np.median(times))
    return {"value": 1.0 / med, "unit": "steps/s", "cores": int(blas or nproc), "kind": "oracle",
            "sample": f"{reps} full steps of all {len(wl.shapes)} matrices (median {med:.2f} s, "
                      f"min {min(times):.2f} s, max {max(times):.2f} s)",
            "nproc": nproc, "cpu_model": model, "blas_threads": blas,
            "seconds_per_step": [round(t, 3) for t in times]}


def after_timed_region(args, plan, grads, total, kw, wl, W, M, work, traffic, dom, fused):
    """Measurements after the timed region: the dominant kernel in a one-stream plan
    (staged plans), a per-iteration coefficient schedule, and the step replayed
    from a HIP graph."""
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

    out = {
        "schedule": {"coeffs": [list(t) for t in sched], "ms_per_step": sched_ms, "steps_per_s": 1000.0 / sched_ms,
                     "note": f"muon_step_schedule, {sched_steps} steps after the timed region"},
        "graph": {"ms_per_step": graph_ms, "steps_per_s": 1000.0 / graph_ms,
                  "note": f"one step captured in a HIP graph, {graph_steps} replays after the timed region"},
    }
    if fused:  # the fused launch already runs alone on one stream
        return out

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
    per_step = p1_cnt / one_steps
    flops = 0 if dom == "momentum" else wl.T * work[dom] / per_step
    roof_one = kernel_roofline(dom, flops, traffic[dom] / per_step, one_ms)
    roof_one.update({"kernel": dom, "ms_per_launch": one_ms,
                     "note": f"one-stream plan (groups=1), {one_steps} steps after the timed region"})

    out["roofline_one_stream"] = roof_one
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--repeats", type=int, default=5, help="times the K-step timed region is run (median reported)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the passes after the timed region (one-stream roofline, schedule, graph)")
    ap.add_argument("--x-master-iters", type=int, default=-1)
    ap.add_argument("--plan", choices=("staged", "fused"), default="staged",
                    help="staged: three launches per iteration on two streams; fused: one persistent launch "
                         "runs every product of the step")
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
    fused = args.plan == "fused"
    plan = MuonStep(W, grads[0], M, x_master_iters=args.x_master_iters, fused=fused)
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
    traffic = traffic_model(wl.shapes, wl.T, 3 if args.x_master_iters < 0 else args.x_master_iters)
    per_kind = {}
    for k, (ms, cnt) in prof_all.items():
        if not cnt:
            continue
        per_kind[k] = {"ms_per_launch": ms / cnt, "launches_per_step": cnt / prof_steps}
        if k in ("gram", "poly", "update"):
            per_kind[k]["tflops"] = wl.T * work[k] / (cnt / prof_steps) / (ms / cnt * 1e-3) / 1e12
            per_kind[k]["gbs"] = traffic[k] / (cnt / prof_steps) / (ms / cnt * 1e-3) / 1e9
        if k == "fused":
            per_kind[k]["tflops"] = work["step"] / (cnt / prof_steps) / (ms / cnt * 1e-3) / 1e12
    if "momentum" in per_kind:
        mk = per_kind["momentum"]
        mk["gbs"] = traffic["momentum"] / mk["launches_per_step"] / (mk["ms_per_launch"] * 1e-3) / 1e9
    dom = max(("gram", "poly", "update", "momentum", "fused"), key=lambda k: prof_all[k][0])

    # timed region: K steps, repeated.  HIP events taken by the library's own
    # launches (on the streams they run on) time the dominant kernel's launches
    # in one step of every `prof_every`: each timed launch delays its stream by
    # a few microseconds, which the other steps do not pay.
    prof_every = 10
    plan.profile(False)
    plan.read_profile()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    rep_ms = []
    prof_steps_timed = 0
    for rep in range(args.repeats):
        torch.cuda.synchronize()
        start.record()
        for t in range(args.warmup, total):
            timed = (t - args.warmup) % prof_every == 0
            if timed:
                plan.profile(True, kinds=[dom])
                prof_steps_timed += 1
            plan.step(grads=grads[t], **kw)
            if timed:
                plan.profile(False)
        stop.record()
        torch.cuda.synchronize()
        rep_ms.append(start.elapsed_time(stop))
    prof = plan.read_profile()
    rep_ms_step = sorted(m / args.steps for m in rep_ms)
    ms_total = sorted(rep_ms)[len(rep_ms) // 2]

    extras = {}
    if not args.no_extras:
        extras = after_timed_region(args, plan, grads, total, kw, wl, W, M, work, traffic, dom, fused)
    plan.close()
    ms_step = ms_total / args.steps
    steps_per_s = 1000.0 / ms_step
    tflops = work["step"] * steps_per_s / 1e12
    d_ms, d_cnt = prof[dom]
    d_launch_ms = d_ms / d_cnt
    d_per_step = d_cnt / prof_steps_timed
    if dom == "momentum":
        roof = kernel_roofline(dom, 0, traffic["momentum"] / d_per_step, d_launch_ms)
    elif dom == "fused":
        nb = traffic["gram"] + traffic["poly"] + traffic["update"]
        roof = kernel_roofline(dom, work["step"] / d_per_step, nb / d_per_step, d_launch_ms)
    else:
        roof = kernel_roofline(dom, wl.T * work[dom] / d_per_step, traffic[dom] / d_per_step, d_launch_ms)
    roof["kernel"] = dom
    roof["scope"] = (f"per launch of the dominant kernel, averaged over its launches in {prof_steps_timed} steps "
                     f"of the timed region (one step in {prof_every})")
    roof["ms_per_launch"] = d_launch_ms
    roof["launches_per_step"] = d_per_step
    roof["traffic"] = read_traffic(dom)
    # share of SIMD cycles with the MFMA unit busy (rocprofv3 counters), when fresh
    roof["mfma_busy"] = read_profile_value("mfma_busy", f"{dom}_mfma_busy")
    roof["step_frac"] = tflops / PEAK_BF16_TFLOPS
    floor_ms = step_floor_ms(work, traffic, wl.T)
    roof["step_roofline"] = {"floor_ms": floor_ms, "measured_ms": ms_step, "frac": floor_ms / ms_step,
                             "note": "sum over the step's launches of the longer of each launch's MFMA and HBM "
                                     "floors (algorithmic FLOPs and bytes at the peaks), over the measured step"}
    if fused:
        roof["note"] = ("the fused launch runs every Newton-Schulz product of the step (all T iterations) on one "
                        "stream; frac is its algorithmic rate over its own duration, step_frac the whole step's "
                        "(momentum and norm included) against the same peak")
    else:
        roof["note"] = ("frac is per launch, against the roof whose floor is longer for the kernel's algorithmic "
                        "FLOPs and bytes (floors_per_launch); the plan runs two matrix groups on two streams, so "
                        "each launch covers half the set and shares the GPU with the other group's launches; "
                        "step_frac is the whole step's algorithmic FLOP rate against the bf16 peak, step_roofline "
                        "the step against the sum of its launches' floors, and roofline_one_stream the kernel's "
                        "own rate without the overlap")

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
                   "lr": wl.lr, "coeffs": list(wl.coeffs), "plan": args.plan},
        "repeats": {"n": args.repeats, "ms_per_step": [round(m, 4) for m in rep_ms_step],
                    "median": rep_ms_step[len(rep_ms_step) // 2], "min": rep_ms_step[0], "max": rep_ms_step[-1],
                    "spread_pct": 100.0 * (rep_ms_step[-1] - rep_ms_step[0]) / rep_ms_step[len(rep_ms_step) // 2],
                    "note": f"the timed region ({args.steps} steps) run {args.repeats} times; value and "
                            "ms_per_step are the median run"},
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
