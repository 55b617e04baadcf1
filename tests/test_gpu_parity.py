"""Parity of the HIP Muon step with the fp64 oracle, through the C ABI (needs an MI355X).

Tolerances (per matrix, per compared step): relative Frobenius error of the
orthogonalised update O <= 2e-2 on the bf16 path and <= 1e-4 on the fp32
path; momentum buffers within 1e-6 * max(1, |M_ref|) elementwise.  O on the
device is recovered from the weight change of that step.
"""
import numpy as np
import pytest
import torch

from muon_harness import (A, B, C, TOL_BF16, TOL_F32, O, check_momentum, compare_run, oracle_steps, run_gpu,
                          say, stream_parity, update_from_weights)
from muon_newton_schulz_03_amd import inputs

pytestmark = pytest.mark.gpu

RAGGED = [(4, 8), (8, 4), (1, 1), (1, 300), (300, 1), (130, 130), (200, 333), (333, 200), (128, 256),
          (257, 129), (77, 1000)]


@pytest.mark.parametrize("path", ["f32", "bf16"])
def test_ragged_shapes(path):
    say(f"[gpu] ragged shapes path={path}")
    gdt = torch.float32 if path == "f32" else torch.bfloat16
    steps = [[inputs.custom_gradient(r, c, 100 * t + i, gdt) for i, (r, c) in enumerate(RAGGED)] for t in range(2)]
    w0 = inputs.weights(RAGGED, seed=5)
    gpu = run_gpu(RAGGED, steps, path=path, lr=0.1, w0=w0)
    worst = compare_run(RAGGED, steps, gpu, path=path, lr=0.1, mu=0.95, nesterov=True, w0=w0)
    say(f"  worst rel err {worst:.3e}")


def test_many_small_matrices_share_blocks():
    """600 small matrices and two large ones, so that blocks run several tiles
    of different K back to back and the ring's requests run ahead across tile
    boundaries; every matrix is compared.  Sides run from 64 to 200: those
    with a short side of 128 or more take the bf16 products (128 x 128 gives
    the Gram product 4 K slabs, the least the ring allows), the others the
    fp32 products in the same step."""
    say("[gpu] many small matrices")
    rng = np.random.default_rng(7)
    sides = [64, 100, 128, 128, 160, 200]
    shapes = [(int(rng.choice(sides)), int(rng.choice(sides))) for _ in range(600)] + [(768, 3072), (256, 1024)]
    steps = [[inputs.custom_gradient(r, c, 1300 + 10 * t + i, std=0.02) for i, (r, c) in enumerate(shapes)]
             for t in range(2)]
    gpu = run_gpu(shapes, steps, path="bf16", lr=0.5)
    worst = compare_run(shapes, steps, gpu, path="bf16", lr=0.5, mu=0.95, nesterov=True)
    say(f"  worst rel err {worst:.3e} over {len(shapes)} matrices")


def test_flat_spectrum():
    """Orthonormal rows or columns: every singular value equal, so all of them
    take the same path through the iteration and any error in the polynomial's
    diagonal moves them all alike.  Stored in bf16 alone, B's diagonal left the
    512-row matrices at about 3e-2 (a CPU emulation of the rounding points);
    with the word per row that keeps it exact, about 9e-3."""
    say("[gpu] flat spectrum")
    shapes = [(512, 4096), (4096, 512), (256, 4096), (768, 768), (1024, 1024), (384, 1536)]
    steps = [[inputs.orthonormal_rows(r, c, 60 + i) for i, (r, c) in enumerate(shapes)]]
    gpu = run_gpu(shapes, steps, path="bf16", lr=0.1)
    worst = compare_run(shapes, steps, gpu, path="bf16", lr=0.1, mu=0.95, nesterov=True)
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


@pytest.mark.timeout(1200)
def test_gpt2_small_ten_steps():
    """72 matrices, 10 consecutive steps with fresh gradients: every matrix is
    compared at every step, and the total weight change after the 10 steps."""
    say("[gpu] gpt2_small 10 steps, all 72 matrices")
    wl = inputs.workload("gpt2_small")
    n = len(wl.shapes)
    res = stream_parity(wl.shapes, lambda t: inputs.gradients("gpt2_small", t), wl.steps,
                        check=lambda t: range(n), track=range(n), lr=wl.lr, mu=wl.momentum)
    assert res.compared == n * wl.steps
    say(f"  worst rel err over {res.compared} (matrix, step) pairs {max(res.worst.values()):.3e}")
    num = den = 0.0
    for i in range(n):  # weights started at zero: W after 10 steps is the total change
        e = O.rel_frobenius(res.w_final[i], res.w_ref[i])
        assert e <= TOL_BF16, f"matrix {i}: total weight change after 10 steps rel err {e:.3e}"
        num += float(np.sum((res.w_final[i] - res.w_ref[i]) ** 2))
        den += float(np.sum(res.w_ref[i] ** 2))
    say(f"  total weight change over the set after 10 steps: rel err {np.sqrt(num / den):.3e}")
    assert np.sqrt(num / den) <= TOL_BF16


QUANTS = (0.0, 0.01, 0.5, 0.99, 1.0)  # min, p1, p50, p99, max


def sigma_quantiles(x: np.ndarray) -> np.ndarray:
    return np.quantile(np.linalg.svd(x, compute_uv=False), QUANTS)


def polar_factor(g: np.ndarray) -> np.ndarray:
    u, _, vt = np.linalg.svd(g, full_matrices=False)
    return u @ vt


@pytest.mark.timeout(900)
def test_illconditioned():
    """24 ill-conditioned 768x768 matrices, one step.  Every output is compared
    with the oracle; the spread of its singular values (min, p1, p50, p99, max)
    is reported and bounded against the oracle's, and its distance to the
    polar factor U V^T of the input is reported beside the oracle's."""
    say("[gpu] illcond768")
    wl = inputs.workload("illcond768")
    steps = [inputs.gradients("illcond768", 0)]
    gpu = run_gpu(wl.shapes, steps, path="bf16", lr=1.0)
    worst = compare_run(wl.shapes, steps, gpu, path="bf16", lr=1.0, mu=0.95, nesterov=True)
    say(f"  worst rel err {worst:.3e}")
    say("  matrix  sigma(gpu) min/p1/p50/p99/max            sigma(oracle) min/p1/p50/p99/max         "
        "rel_F to UV^T gpu / oracle")
    dq_worst = 0.0
    for i in range(len(wl.shapes)):
        og = update_from_weights(gpu.W[0][i], np.zeros(wl.shapes[i]), 1.0)
        ref = oracle_steps(torch.zeros(wl.shapes[i]), [steps[0][i]], lr=1.0)[0].O
        qg, qr = sigma_quantiles(og), sigma_quantiles(ref)
        # the first Nesterov step from zero momentum orthogonalises (1 + mu) G: U V^T of G
        uv = polar_factor(O.as_f64(steps[0][i]))
        dg, dr = O.rel_frobenius(og, uv), O.rel_frobenius(ref, uv)
        say(f"  {i:6d}  " + " ".join(f"{v:.4f}" for v in qg) + "   " + " ".join(f"{v:.4f}" for v in qr)
            + f"   {dg:.4f} / {dr:.4f}")
        # singular values of nearby matrices differ by at most the spectral norm of the
        # difference (Weyl), which the Frobenius distance bounds; the band the quintic
        # targets is of unit scale, so each quantile must also agree within TOL_BF16
        e = O.rel_frobenius(og, ref)
        assert np.max(np.abs(qg - qr)) <= e * np.linalg.norm(ref) + 1e-9, (i, qg, qr)
        assert np.max(np.abs(qg - qr)) <= TOL_BF16, (i, qg, qr)
        assert abs(dg - dr) <= e * np.linalg.norm(ref) / np.linalg.norm(uv) + 1e-9
        dq_worst = max(dq_worst, float(np.max(np.abs(qg - qr))))
    say(f"  largest sigma-quantile difference gpu vs oracle {dq_worst:.3e}")


@pytest.mark.timeout(900)
@pytest.mark.parametrize("nesterov", [True, False])
def test_aspect_ratio_transpose(nesterov):
    """48 matrices alternating 3072x768 / 768x3072: all 48 compared at the
    third step, two of each orientation at every step."""
    say(f"[gpu] aspect3072 nesterov={nesterov}")
    wl = inputs.workload("aspect3072")
    run = 0 if nesterov else 1
    n = len(wl.shapes)
    last = wl.steps - 1
    res = stream_parity(wl.shapes, lambda t: inputs.gradients("aspect3072", t, run=run), wl.steps,
                        check=lambda t: range(n) if t == last else [0, 1, 46, 47], lr=1.0, nesterov=nesterov)
    assert len(res.worst) == n
    say(f"  worst rel err {max(res.worst.values()):.3e} over {res.compared} (matrix, step) pairs")


@pytest.mark.timeout(1200)
def test_width1024_fifty_steps():
    """144 matrices, 50 steps with the state kept on device: matrices of every
    shape from both plan groups (layers 0 and 23) compared at steps 1, 2, 10, 25
    and 50, and the weights of one matrix per group after all 50 steps."""
    say("[gpu] width1024 50 steps")
    wl = inputs.workload("width1024")
    from muon_newton_schulz_03_amd.muon import describe
    info, _ = describe(wl.shapes)
    assert info["n_groups"] == 2
    check_steps = {0, 1, 9, 24, 49}
    sample = [0, 4, 5, 72, 76, 77, 142, 143]
    track = [0, 143]
    res = stream_parity(wl.shapes, lambda t: inputs.gradients("width1024", t, device="cuda:0"), wl.steps,
                        check=lambda t: sample if t in check_steps else [], track=track, lr=wl.lr)
    assert sorted(res.worst) == sample and res.compared == len(sample) * len(check_steps)
    say("  worst rel err per matrix: " + ", ".join(f"{i}: {res.worst[i]:.2e}" for i in sample))
    for i in track:
        e = O.rel_frobenius(res.w_final[i], res.w_ref[i])
        say(f"  matrix {i} {wl.shapes[i]} weights after 50 steps rel err {e:.3e}")
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


@pytest.mark.parametrize("fused", [False, True])
def test_later_work_on_the_stream_sees_the_whole_step(fused):
    """Work enqueued on the caller's stream right after a step (no host
    synchronisation) reads every matrix's final weights and momentum: the
    first group runs on that stream, the second forks from it and joins back
    (the staged plan); the fused plan runs there alone.  Both groups of
    GPT-2 small, three steps in a row before the snapshot."""
    say(f"[gpu] stream order after a step, fused={fused}")
    from muon_newton_schulz_03_amd import MuonStep
    wl = inputs.workload("gpt2_small")
    dev = torch.device("cuda:0")
    grads = [inputs.gradients("gpt2_small", t, device=dev) for t in range(3)]
    W = [torch.zeros(s, device=dev) for s in wl.shapes]
    M = [torch.zeros(s, device=dev) for s in wl.shapes]
    plan = MuonStep(W, grads[0], M, fused=fused)
    torch.cuda.synchronize()
    for t in range(3):
        plan.step(grads=grads[t], lr=wl.lr, momentum=wl.momentum)
    snap_w = [w.clone() for w in W]  # same stream, queued behind the steps
    snap_m = [m.clone() for m in M]
    torch.cuda.synchronize()
    for i in range(len(W)):
        assert torch.equal(snap_w[i], W[i]) and torch.equal(snap_m[i], M[i]), f"matrix {i}"
        assert torch.count_nonzero(W[i]).item() > 0, f"matrix {i} was not updated"
    plan.close()


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
    # the oracle over the same four steps (the gradient buffers keep their values)
    refs = [oracle_steps(torch.zeros(s), [G[i].cpu()] * 4, lr=kw["lr"]) for i, s in enumerate(shapes)]
    prev = [np.zeros(s) for s in shapes]
    for rep in range(4):
        pe.step(**kw)
        graph.replay()
        scratch = torch.randn(1 << 20, device=dev).sum()  # eager work between replays
        torch.cuda.synchronize()
        for i in range(len(shapes)):
            assert torch.equal(We[i], Wg[i]) and torch.equal(Me[i], Mg[i]), f"replay {rep} matrix {i}"
            w = Wg[i].cpu().double().numpy()
            e = O.rel_frobenius(update_from_weights(w, prev[i], kw["lr"]), refs[i][rep].O)
            assert e <= TOL_BF16, f"replay {rep} matrix {i}: rel err {e:.3e} against the oracle"
            check_momentum(Mg[i].cpu(), refs[i][rep].M, f"replay {rep} matrix {i}")
            prev[i] = w
        assert torch.isfinite(scratch)
    # the captured plan's pointers are fixed: new buffers are refused, eagerly and under capture
    from muon_newton_schulz_03_amd._lib import MUON_E_INVAL, MuonError
    other = [torch.zeros(s, device=dev) for s in shapes]
    with pytest.raises(MuonError, match="captured") as err:
        pg.step(weights=other, **kw)
    assert err.value.code == MUON_E_INVAL
    g2 = torch.cuda.CUDAGraph()
    with pytest.raises(MuonError, match="capturing"):
        with torch.cuda.graph(g2):
            torch.ones(4, device=dev).mul_(2)  # the graph is not empty when the step is refused
            pe.step(weights=other, **kw)
    torch.cuda.synchronize()
    pe.close()
    pg.close()


def test_nan_gradient_stays_in_its_matrix():
    """A NaN in one gradient reaches that matrix's momentum (at that entry only)
    and its weights; every other matrix of the plan is bitwise unchanged."""
    say("[gpu] NaN gradient isolation")
    shapes = [(256, 384), (384, 256), (200, 200), (768, 768)]
    clean = [[inputs.custom_gradient(r, c, 1200 + i) for i, (r, c) in enumerate(shapes)]]
    bad = [[g.clone() for g in clean[0]]]
    bad[0][1][17, 5] = float("nan")
    for groups in (1, 2):
        ref = run_gpu(shapes, clean, lr=0.1, groups=groups)
        got = run_gpu(shapes, bad, lr=0.1, groups=groups)
        for i in (0, 2, 3):
            assert torch.equal(got.W[0][i], ref.W[0][i]) and torch.equal(got.M[0][i], ref.M[0][i]), (groups, i)
        m_nan = torch.isnan(got.M[0][1])
        assert m_nan[17, 5] and int(m_nan.sum()) == 1
        keep = ~m_nan
        assert torch.equal(got.M[0][1][keep], ref.M[0][1][keep])
        assert torch.isnan(got.W[0][1]).all()
