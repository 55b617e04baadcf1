"""Parity of the HIP Muon step with the fp64 oracle, through the C ABI (needs an MI355X).

Tolerances (per matrix, per compared step): relative Frobenius error of the
orthogonalised update O <= 2e-2 on the bf16 path and <= 1e-4 on the fp32
path; momentum buffers within 1e-6 * max(1, |M_ref|) elementwise.  O on the
device is recovered from the weight change of that step.
"""
import numpy as np
import pytest
import torch

from muon_harness import (A, B, C, TOL_BF16, TOL_F32, O, check_momentum, oracle_steps, run_gpu, say,
                          update_from_weights)
from muon_newton_schulz_03_amd import inputs

pytestmark = pytest.mark.gpu

RAGGED = [(4, 8), (8, 4), (1, 1), (1, 300), (300, 1), (130, 130), (200, 333), (333, 200), (128, 256),
          (257, 129), (77, 1000)]


def compare_run(shapes, grads_steps, gpu, *, path, lr, mu, nesterov, T=5, coeffs=(A, B, C), w0=None,
                scales=None, sample=None, steps=None, tol=None, schedule=None):
    tol = tol if tol is not None else (TOL_F32 if path == "f32" else TOL_BF16)
    sample = list(range(len(shapes))) if sample is None else list(sample)
    worst = 0.0
    for si, i in enumerate(sample):
        wi0 = w0[i] if w0 is not None else torch.zeros(shapes[i])
        s = 1.0 if scales is None or scales[i] <= 0 else O.f32(scales[i])
        ref = oracle_steps(wi0, [g[i] for g in grads_steps], T=T, mu=mu, nesterov=nesterov, lr=lr,
                           coeffs=coeffs, scale=s, schedule=schedule)
        prev = O.as_f64(wi0)
        for t, r in enumerate(ref):
            if gpu.W[t] is None or (t > 0 and gpu.W[t - 1] is None):
                continue
            og = update_from_weights(gpu.W[t][si], prev if t == 0 else gpu.W[t - 1][si], lr, s)
            e = O.rel_frobenius(og, r.O)
            worst = max(worst, e)
            assert e <= tol, f"matrix {i} {shapes[i]} step {t}: rel err {e:.3e} > {tol}"
            check_momentum(gpu.M[t][si], r.M, f"matrix {i} step {t}")
    return worst


@pytest.mark.parametrize("path", ["f32", "bf16"])
def test_ragged_shapes(path):
    say(f"[gpu] ragged shapes path={path}")
    gdt = torch.float32 if path == "f32" else torch.bfloat16
    steps = [[inputs.custom_gradient(r, c, 100 * t + i, gdt) for i, (r, c) in enumerate(RAGGED)] for t in range(2)]
    w0 = inputs.weights(RAGGED, seed=5)
    gpu = run_gpu(RAGGED, steps, path=path, lr=0.1, w0=w0)
    worst = compare_run(RAGGED, steps, gpu, path=path, lr=0.1, mu=0.95, nesterov=True, w0=w0)
    say(f"  worst rel err {worst:.3e}")


def test_single768_fp32():
    say("[gpu] single768 fp32 path")
    wl = inputs.workload("single768")
    steps = [inputs.gradients("single768", 0)]
    gpu = run_gpu(wl.shapes, steps, path="f32", lr=wl.lr)
    worst = compare_run(wl.shapes, steps, gpu, path="f32", lr=wl.lr, mu=0.95, nesterov=True)
    say(f"  rel err {worst:.3e}")
    assert worst <= TOL_F32


def test_single768_bf16_path_too():
    say("[gpu] single768 through the bf16 path")
    steps = [[g.to(torch.bfloat16) for g in inputs.gradients("single768", 0)]]
    gpu = run_gpu([(768, 768)], steps, path="bf16", lr=1.0)
    worst = compare_run([(768, 768)], steps, gpu, path="bf16", lr=1.0, mu=0.95, nesterov=True)
    say(f"  rel err {worst:.3e}")


def test_gpt2_small_ten_steps():
    """72 matrices, 10 consecutive steps; one layer's six matrices checked at every step."""
    say("[gpu] gpt2_small 10 steps")
    wl = inputs.workload("gpt2_small")
    steps = [inputs.gradients("gpt2_small", t) for t in range(wl.steps)]
    sample = [0, 3, 4, 5, 66, 71]
    gpu = run_gpu(wl.shapes, steps, path="bf16", lr=wl.lr, sample=sample)
    worst = compare_run(wl.shapes, steps, gpu, path="bf16", lr=wl.lr, mu=wl.momentum, nesterov=True,
                        sample=sample)
    say(f"  worst rel err {worst:.3e}")


def test_illconditioned():
    say("[gpu] illcond768")
    wl = inputs.workload("illcond768")
    steps = [inputs.gradients("illcond768", 0)]
    gpu = run_gpu(wl.shapes, steps, path="bf16", lr=1.0)
    worst = compare_run(wl.shapes, steps, gpu, path="bf16", lr=1.0, mu=0.95, nesterov=True)
    say(f"  worst rel err {worst:.3e}")
    # singular-value spread of one output: same band as the oracle's
    og = update_from_weights(gpu.W[0][0], np.zeros((768, 768)), 1.0)
    ref = oracle_steps(torch.zeros(768, 768), [steps[0][0]], lr=1.0)[0].O
    sg, sr = np.linalg.svd(og, compute_uv=False), np.linalg.svd(ref, compute_uv=False)
    say(f"  sigma gpu [{sg.min():.4f}, {np.median(sg):.4f}, {sg.max():.4f}]"
        f" oracle [{sr.min():.4f}, {np.median(sr):.4f}, {sr.max():.4f}]")
    assert abs(sg.max() - sr.max()) < 0.02 and abs(np.median(sg) - np.median(sr)) < 0.02


@pytest.mark.parametrize("nesterov", [True, False])
def test_aspect_ratio_transpose(nesterov):
    say(f"[gpu] aspect3072 nesterov={nesterov}")
    wl = inputs.workload("aspect3072")
    run = 0 if nesterov else 1
    steps = [inputs.gradients("aspect3072", t, run=run) for t in range(wl.steps)]
    sample = [0, 1, 46, 47]
    gpu = run_gpu(wl.shapes, steps, path="bf16", lr=1.0, nesterov=nesterov, sample=sample)
    worst = compare_run(wl.shapes, steps, gpu, path="bf16", lr=1.0, mu=0.95, nesterov=nesterov, sample=sample)
    say(f"  worst rel err {worst:.3e}")


def test_width1024_fifty_steps():
    """144 matrices, 50 steps with state kept on device; sampled matrices checked at
    steps 1, 2, 10, 25, 50 and the weight change of one matrix after all 50."""
    say("[gpu] width1024 50 steps")
    wl = inputs.workload("width1024")
    dev = "cuda:0"
    check_steps = {0, 1, 9, 24, 49}
    sample = [0, 4, 5]
    steps = [inputs.gradients("width1024", t, device=dev) for t in range(wl.steps)]
    keep = sorted(check_steps | {t - 1 for t in check_steps if t > 0})
    gpu = run_gpu(wl.shapes, steps, path="bf16", lr=wl.lr, sample=sample, keep_steps=keep)
    for si, i in enumerate(sample):
        say(f"  oracle for matrix {i} {wl.shapes[i]}")
        grads = [steps[t][i].cpu() for t in range(wl.steps)]
        need = check_steps if si > 0 else None  # matrix 0: the full 50-step oracle
        ref = oracle_steps(torch.zeros(wl.shapes[i]), grads, lr=wl.lr, need_ns=need)
        for t in sorted(check_steps):
            prev = np.zeros(wl.shapes[i]) if t == 0 else gpu.W[t - 1][si]
            og = update_from_weights(gpu.W[t][si], prev, wl.lr)
            e = O.rel_frobenius(og, ref[t].O)
            assert e <= TOL_BF16, f"matrix {i} step {t}: {e:.3e}"
            check_momentum(gpu.M[t][si], ref[t].M, f"matrix {i} step {t}")
        if si == 0:
            e = O.rel_frobenius(-gpu.W[49][0], -ref[49].W)
            say(f"  matrix 0 weight after 50 steps rel err {e:.3e}")
            assert e <= TOL_BF16


def test_determinism_and_grouping():
    """Bitwise: two runs agree, a grouped plan equals one plan per matrix, and the
    two-stream plan equals the one-stream plan."""
    say("[gpu] determinism / grouped launch")
    shapes = [(256, 384), (384, 256), (200, 200)]
    steps = [[inputs.custom_gradient(r, c, 500 + 10 * t + i) for i, (r, c) in enumerate(shapes)] for t in range(3)]
    g1 = run_gpu(shapes, steps, lr=0.1)
    g2 = run_gpu(shapes, steps, lr=0.1)
    for t in range(3):
        for i in range(3):
            assert torch.equal(g1.W[t][i], g2.W[t][i]) and torch.equal(g1.M[t][i], g2.M[t][i])
    for i in range(3):
        single = run_gpu([shapes[i]], [[s[i]] for s in steps], lr=0.1)
        for t in range(3):
            assert torch.equal(single.W[t][0], g1.W[t][i])
    one = run_gpu(shapes, steps, lr=0.1, groups=1)
    for t in range(3):
        for i in range(3):
            assert torch.equal(one.W[t][i], g1.W[t][i]) and torch.equal(one.M[t][i], g1.M[t][i])


def test_resume_equals_straight_run():
    say("[gpu] resume 2+2 == 4")
    from muon_newton_schulz_03_amd import MuonStep
    dev = "cuda:0"
    shapes = [(256, 512), (512, 256)]
    steps = [[inputs.custom_gradient(r, c, 900 + 10 * t + i).to(dev) for i, (r, c) in enumerate(shapes)]
             for t in range(4)]

    def fresh():
        return ([torch.zeros(s, device=dev) for s in shapes], [torch.zeros(s, device=dev) for s in shapes])

    W, M = fresh()
    G = [g.clone() for g in steps[0]]
    p = MuonStep(W, G, M)
    for t in range(4):
        for i in range(2):
            G[i].copy_(steps[t][i])
        p.step(lr=0.1)
    torch.cuda.synchronize()
    p.close()
    W2, M2 = fresh()
    for half in (0, 2):
        p = MuonStep(W2, G, M2)  # a new plan over the saved state
        for t in (half, half + 1):
            for i in range(2):
                G[i].copy_(steps[t][i])
            p.step(lr=0.1)
        torch.cuda.synchronize()
        p.close()
    for i in range(2):
        assert torch.equal(W[i], W2[i]) and torch.equal(M[i], M2[i])


@pytest.mark.parametrize("path", ["bf16", "f32"])
def test_zero_iterations(path):
    say(f"[gpu] T=0 path={path}")
    shapes = [(96, 160), (160, 96)]
    gdt = torch.float32 if path == "f32" else torch.bfloat16
    steps = [[inputs.custom_gradient(r, c, 40 + i, gdt) for i, (r, c) in enumerate(shapes)]]
    gpu = run_gpu(shapes, steps, path=path, T=0, lr=0.5)
    compare_run(shapes, steps, gpu, path=path, T=0, lr=0.5, mu=0.95, nesterov=True, tol=1e-5)


def test_other_coefficients_and_scales():
    """Convergent coefficients reach the polar factor; per-matrix scales and bf16 weights."""
    say("[gpu] coefficients / scales / bf16 weights")
    shapes = [(128, 384), (384, 128)]
    rng = np.random.default_rng(3)
    grads = []
    for r, c in shapes:
        u, _ = np.linalg.qr(rng.standard_normal((r, min(r, c))))
        v, _ = np.linalg.qr(rng.standard_normal((c, min(r, c))))
        s = np.linspace(1.0, 0.25, min(r, c))
        grads.append(torch.from_numpy((u * s) @ v.T).float())
    steps = [grads]
    coeffs = (15 / 8, -10 / 8, 3 / 8)
    gpu = run_gpu(shapes, steps, path="f32", T=12, coeffs=coeffs, lr=1.0, scales=[2.0, 0.5], mu=0.0)
    compare_run(shapes, steps, gpu, path="f32", T=12, coeffs=coeffs, lr=1.0, mu=0.0, nesterov=True,
                scales=[2.0, 0.5])
    for i in range(2):
        og = update_from_weights(gpu.W[0][i], np.zeros(shapes[i]), 1.0, [2.0, 0.5][i])
        u, _, vt = np.linalg.svd(grads[i].double().numpy(), full_matrices=False)
        assert O.rel_frobenius(og, u @ vt) < 1e-4
    # bf16 weights: the step is applied with one bf16 rounding of W
    w0 = [torch.full(s, 0.5) for s in shapes]
    bgpu = run_gpu(shapes, [[g.bfloat16() for g in grads]], lr=0.01, w0=w0, weight_dtype=torch.bfloat16)
    for i in range(2):
        ref = oracle_steps(w0[i], [grads[i].bfloat16()], lr=0.01)[0]
        assert np.max(np.abs(bgpu.W[0][i].numpy() - ref.W)) <= 2 ** -8 * 0.5 + 0.01 * 0.02 * np.abs(ref.O).max()


def test_zero_gradient_and_pointer_change():
    say("[gpu] zero gradient / new tensors at step")
    from muon_newton_schulz_03_amd import MuonStep
    dev = "cuda:0"
    shapes = [(64, 96)]
    W = [torch.ones(shapes[0], device=dev)]
    M = [torch.zeros(shapes[0], device=dev)]
    G = [torch.zeros(shapes[0], device=dev, dtype=torch.bfloat16)]
    p = MuonStep(W, G, M)
    p.step(lr=0.1)
    torch.cuda.synchronize()
    assert torch.equal(W[0], torch.ones_like(W[0])) and not torch.isnan(W[0]).any()
    # new weight/grad/momentum tensors at step time
    g = inputs.custom_gradient(64, 96, 77).to(dev)
    W2, M2 = [torch.zeros(shapes[0], device=dev)], [torch.zeros(shapes[0], device=dev)]
    p.step(lr=0.1, weights=W2, grads=[g], moms=M2)
    torch.cuda.synchronize()
    ref = oracle_steps(torch.zeros(shapes[0]), [g.cpu()], lr=0.1)[0]
    assert O.rel_frobenius(W2[0].cpu().double().numpy(), ref.W) < TOL_BF16
    assert torch.equal(W[0], torch.ones_like(W[0]))
    p.close()


def test_profile_counts():
    say("[gpu] profiling")
    from muon_newton_schulz_03_amd import MuonStep
    dev = "cuda:0"
    shapes = [(256, 256), (256, 1024)]
    W = [torch.zeros(s, device=dev) for s in shapes]
    M = [torch.zeros(s, device=dev) for s in shapes]
    G = [inputs.custom_gradient(r, c, 3).to(dev) for r, c in shapes]
    p = MuonStep(W, G, M)
    from muon_newton_schulz_03_amd.muon import describe
    groups = describe(shapes)[0]["n_groups"]
    assert groups == 2  # two matrices: one per group stream
    p.profile(True)
    for _ in range(3):
        p.step(T=5)
    prof = p.read_profile()
    assert prof["momentum"][1] == 3 * groups and prof["gram"][1] == 15 * groups and prof["update"][1] == 15 * groups
    assert all(prof[k][0] > 0 for k in ("momentum", "gram", "poly", "update"))
    # only the selected kind is timed
    p.profile(True, kinds=["update"])
    p.step(T=5)
    prof = p.read_profile()
    assert prof["update"][1] == 5 * groups and prof["gram"][1] == 0 and prof["momentum"][1] == 0
    p.close()


@pytest.mark.parametrize("k", [0, 5])
def test_master_copy_settings(k):
    """x_master_iters = 0 (bf16 X throughout) and 5 (the (bf16, low byte) pair every iteration) also pass."""
    say(f"[gpu] x_master_iters={k}")
    shapes = [(768, 768)] * 2 + [(768, 3072)]
    steps = [[inputs.custom_gradient(r, c, 60 + i, std=0.02) for i, (r, c) in enumerate(shapes)]]
    gpu = run_gpu(shapes, steps, lr=1.0, x_master_iters=k)
    worst = compare_run(shapes, steps, gpu, path="bf16", lr=1.0, mu=0.95, nesterov=True)
    say(f"  worst rel err {worst:.3e}")


# per-iteration coefficient schedules (muon_step_schedule): an aggressive start
# with the speedrun quintic, then other polynomials, a convergent quintic last
SCHED5 = [(A, B, C), (A, B, C), (3.0, -3.2, 1.2), (15 / 8, -10 / 8, 3 / 8), (1.5, -0.5, 0.0)]
SCHED8 = [(A, B, C)] * 3 + [(15 / 8, -10 / 8, 3 / 8)] * 5


@pytest.mark.parametrize("path,sched", [("bf16", SCHED5), ("bf16", SCHED8), ("f32", SCHED5)])
def test_schedule_parity(path, sched):
    say(f"[gpu] schedule path={path} T={len(sched)}")
    gdt = torch.float32 if path == "f32" else torch.bfloat16
    shapes = [(256, 384), (384, 256), (768, 768), (100, 37)]
    steps = [[inputs.custom_gradient(r, c, 700 + 10 * t + i, gdt, std=0.02) for i, (r, c) in enumerate(shapes)]
             for t in range(2)]
    gpu = run_gpu(shapes, steps, path=path, lr=0.5, schedule=sched)
    worst = compare_run(shapes, steps, gpu, path=path, lr=0.5, mu=0.95, nesterov=True, schedule=sched)
    say(f"  worst rel err {worst:.3e}")


def test_schedule_of_one_triple_equals_plain_step():
    say("[gpu] uniform schedule == muon_step")
    shapes = [(256, 512), (512, 256)]
    steps = [[inputs.custom_gradient(r, c, 800 + 10 * t + i) for i, (r, c) in enumerate(shapes)] for t in range(2)]
    plain = run_gpu(shapes, steps, lr=0.1)
    sched = run_gpu(shapes, steps, lr=0.1, schedule=[(A, B, C)] * 5)
    for t in range(2):
        for i in range(2):
            assert torch.equal(plain.W[t][i], sched.W[t][i]) and torch.equal(plain.M[t][i], sched.M[t][i])


@pytest.mark.parametrize("groups", [1, 2])
def test_graph_capture_replays_match_eager(groups):
    """A step captured in a graph (descriptors unchanged, profiling off), replayed
    several times with eager work and synchronisation in between, gives the eager
    run's weights and momentum bitwise after every replay."""
    say(f"[gpu] graph capture groups={groups}")
    from muon_newton_schulz_03_amd import MuonStep
    dev = "cuda:0"
    shapes = [(256, 384), (384, 256), (128, 640)]
    G = [inputs.custom_gradient(r, c, 950 + i).to(dev) for i, (r, c) in enumerate(shapes)]
    kw = dict(T=5, momentum=0.95, nesterov=True, lr=0.1)

    We = [torch.zeros(s, device=dev) for s in shapes]
    Me = [torch.zeros(s, device=dev) for s in shapes]
    pe = MuonStep(We, G, Me, groups=groups)
    Wg = [torch.zeros(s, device=dev) for s in shapes]
    Mg = [torch.zeros(s, device=dev) for s in shapes]
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        pg = MuonStep(Wg, G, Mg, groups=groups)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        pg.step(**kw)  # captured, not run
    torch.cuda.synchronize()
    for w in Wg + Mg:
        assert torch.count_nonzero(w).item() == 0  # capture ran nothing
    for rep in range(4):
        pe.step(**kw)
        graph.replay()
        scratch = torch.randn(1 << 20, device=dev).sum()  # eager work between replays
        torch.cuda.synchronize()
        for i in range(len(shapes)):
            assert torch.equal(We[i], Wg[i]) and torch.equal(Me[i], Mg[i]), f"replay {rep} matrix {i}"
        assert torch.isfinite(scratch)
    pe.close()
    pg.close()
