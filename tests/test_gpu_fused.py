"""Fused plans on the GPU: one persistent launch per step runs every bf16
product, blocks taking their XCD's tiles in order and waiting on per-matrix
counters.  It runs the same tiles with the same arithmetic as the three
launches per iteration, so weights and momentum must come out bitwise equal
to the staged plan's; the oracle bounds both.
"""
import numpy as np
import pytest
import torch

from muon_harness import A, B, C, TOL_BF16, O, check_momentum, oracle_steps, say, update_from_weights
from muon_newton_schulz_03_amd import inputs

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def run_plan(shapes, grads_steps, *, fused, w0=None, weight_dtype=torch.float32, steps_kw=None, **kw):
    """Weights and momentum (CPU copies) after each step of one plan."""
    from muon_newton_schulz_03_amd import MuonStep
    W = [(torch.zeros(s) if w0 is None else w0[i]).to(DEV, weight_dtype).contiguous() for i, s in enumerate(shapes)]
    M = [torch.zeros(s, device=DEV) for s in shapes]
    G = [g.to(DEV).clone() for g in grads_steps[0]]
    plan = MuonStep(W, G, M, fused=fused)
    out = []
    for t, grads in enumerate(grads_steps):
        if t > 0:
            for i in range(len(shapes)):
                G[i].copy_(grads[i].to(DEV))
        step_kw = dict(kw)
        if steps_kw is not None:
            step_kw.update(steps_kw[t])
        plan.step(**step_kw)
        plan.check()
        torch.cuda.synchronize()
        out.append(([w.cpu().clone() for w in W], [m.cpu().clone() for m in M]))
    plan.close()
    return out


def assert_bitwise(a, b, what):
    for t, ((wa, ma), (wb, mb)) in enumerate(zip(a, b)):
        for i in range(len(wa)):
            assert torch.equal(wa[i], wb[i]), f"{what}: step {t} matrix {i}: weights differ"
            assert torch.equal(ma[i], mb[i]), f"{what}: step {t} matrix {i}: momentum differs"


def test_fused_plan_is_fused():
    from muon_newton_schulz_03_amd import MuonStep
    shapes = [(256, 512), (64, 64)]
    W = [torch.zeros(s, device=DEV) for s in shapes]
    M = [torch.zeros(s, device=DEV) for s in shapes]
    G = [inputs.custom_gradient(r, c, 7 + i).to(DEV) for i, (r, c) in enumerate(shapes)]
    plan = MuonStep(W, G, M, fused=True)
    plan.profile(True)
    plan.step(T=5)
    plan.check()
    prof = plan.read_profile()
    assert prof["fused"][1] == 1 and prof["gram"][1] == 5 and prof["update"][1] == 5  # the 64 x 64 one: fp32 launches
    plan.step(T=17)  # beyond the launch's coefficient slots: three launches per iteration
    plan.check()
    prof = plan.read_profile()
    assert prof["fused"][1] == 0 and prof["gram"][1] == 2 * 17
    plan.close()


def test_fused_matches_staged_gpt2_small():
    """The 72 hidden matrices of GPT-2 small, three steps with fresh gradients:
    bitwise equal to the staged plan, and every matrix of the first step
    within the bf16 tolerance of the oracle."""
    say("[gpu] fused vs staged, gpt2_small, 3 steps")
    wl = inputs.workload("gpt2_small")
    steps = [inputs.gradients("gpt2_small", t) for t in range(3)]
    kw = dict(T=5, momentum=wl.momentum, nesterov=True, lr=wl.lr)
    staged = run_plan(wl.shapes, steps, fused=False, **kw)
    fused = run_plan(wl.shapes, steps, fused=True, **kw)
    assert_bitwise(staged, fused, "gpt2_small")
    worst = 0.0
    for i, s in enumerate(wl.shapes):
        r = oracle_steps(torch.zeros(s), [steps[0][i]], lr=wl.lr, mu=wl.momentum)[0]
        e = O.rel_frobenius(update_from_weights(fused[0][0][i].double().numpy(), np.zeros(s), wl.lr), r.O)
        worst = max(worst, e)
        assert e <= TOL_BF16, f"matrix {i} {s}: rel err {e:.3e}"
        check_momentum(fused[0][1][i], r.M, f"matrix {i}")
    say(f"  bitwise equal over 3 steps; worst rel err against the oracle {worst:.3e}")


RAGGED_MIX = [(300, 700), (700, 300), (129, 4100), (1000, 130), (64, 64), (100, 333), (256, 256), (512, 1536),
              (1536, 512), (384, 384)]


def test_fused_ragged_mixed_precisions_bf16_weights():
    """Ragged shapes, matrices that take the fp32 products beside the fused
    launch, fp32 and bf16 weights: bitwise equal to the staged plan, and the
    fp32-weight run within the tolerance of the oracle."""
    say("[gpu] fused vs staged, ragged and mixed")
    shapes = RAGGED_MIX
    steps = [[inputs.custom_gradient(r, c, 4100 + 10 * t + i) for i, (r, c) in enumerate(shapes)] for t in range(2)]
    w0 = inputs.weights(shapes, seed=41)
    kw = dict(T=5, momentum=0.9, nesterov=False, lr=0.2)
    runs = {}
    for wdt in (torch.float32, torch.bfloat16):
        staged = run_plan(shapes, steps, fused=False, w0=w0, weight_dtype=wdt, **kw)
        runs[wdt] = run_plan(shapes, steps, fused=True, w0=w0, weight_dtype=wdt, **kw)
        assert_bitwise(staged, runs[wdt], f"ragged {wdt}")
    fused = runs[torch.float32]
    worst = 0.0
    for i, s in enumerate(shapes):
        ref = oracle_steps(w0[i], [st[i] for st in steps], lr=kw["lr"], mu=kw["momentum"], nesterov=False)
        prev = O.as_f64(w0[i])
        for t in range(2):
            w = fused[t][0][i].double().numpy()
            e = O.rel_frobenius(update_from_weights(w, prev, kw["lr"]), ref[t].O)
            worst = max(worst, e)
            assert e <= TOL_BF16, f"matrix {i} {s} step {t}: rel err {e:.3e}"
            prev = w
    say(f"  bitwise equal (fp32 and bf16 weights); worst rel err {worst:.3e}")


def test_fused_schedules_and_iteration_counts():
    """Per-iteration coefficients and T = 1, 3, 16 (the launch's limit) and
    17 (staged fallback): bitwise equal to the staged plan."""
    say("[gpu] fused vs staged, schedules and T")
    shapes = [(768, 768), (768, 3072), (3072, 768), (512, 1024)]
    steps = [[inputs.custom_gradient(r, c, 5200 + i) for i, (r, c) in enumerate(shapes)]]
    sched = [(A, B, C)] * 3 + [(1.875, -1.25, 0.375)] * 3
    for skw in (dict(schedule=sched), dict(T=1), dict(T=3), dict(T=16), dict(T=17)):
        kw = dict(momentum=0.95, nesterov=True, lr=0.05, **skw)
        staged = run_plan(shapes, steps, fused=False, **kw)
        fused = run_plan(shapes, steps, fused=True, **kw)
        assert_bitwise(staged, fused, f"{skw if 'T' in skw else 'schedule'}")
    say("  bitwise equal for the schedule and T = 1, 3, 16, 17")


def test_fused_wait_gives_up_and_recovers():
    """A wait whose target is never met gives up after its poll limit: every
    block returns, the launch ends, muon_check reports it (MUON_E_HIP) and
    clears the report; the plan then steps normally again."""
    say("[gpu] fused: bounded waits give up")
    from muon_newton_schulz_03_amd import MuonStep
    from muon_newton_schulz_03_amd._lib import MUON_E_HIP, MuonError
    shapes = [(768, 768), (768, 3072)]
    W = [torch.zeros(s, device=DEV) for s in shapes]
    M = [torch.zeros(s, device=DEV) for s in shapes]
    G = [inputs.custom_gradient(r, c, 61 + i).to(DEV) for i, (r, c) in enumerate(shapes)]
    plan = MuonStep(W, G, M, fused=True)
    plan.fused_limits(spin_limit=64, dep_bias=1 << 30)
    plan.step(T=5, lr=0.1)
    with pytest.raises(MuonError, match="gave up") as err:
        plan.check()
    assert err.value.code == MUON_E_HIP
    torch.cuda.synchronize()
    assert all(torch.count_nonzero(w).item() == 0 for w in W)  # no tile ran: weights untouched
    plan.check()  # the report was cleared
    plan.fused_limits(spin_limit=1 << 24, dep_bias=0)
    plan.step(T=5, lr=0.1)
    plan.check()
    torch.cuda.synchronize()
    assert all(torch.count_nonzero(w).item() > 0 for w in W)
    plan.close()
    say("  gave up, reported, recovered")


def test_fused_step_in_a_graph():
    """A fused step captured in a HIP graph and replayed (eager work and
    synchronisation between replays) matches the eager fused plan bitwise
    after every replay; the counters the launch waits on are reset by the
    norm launch inside the graph."""
    say("[gpu] fused step in a graph")
    from muon_newton_schulz_03_amd import MuonStep
    shapes = [(768, 768), (768, 3072), (512, 256), (64, 64)]
    G = [inputs.custom_gradient(r, c, 7300 + i).to(DEV) for i, (r, c) in enumerate(shapes)]
    kw = dict(T=5, momentum=0.95, nesterov=True, lr=0.1)
    We = [torch.zeros(s, device=DEV) for s in shapes]
    Me = [torch.zeros(s, device=DEV) for s in shapes]
    pe = MuonStep(We, G, Me, fused=True)
    Wg = [torch.zeros(s, device=DEV) for s in shapes]
    Mg = [torch.zeros(s, device=DEV) for s in shapes]
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        pg = MuonStep(Wg, G, Mg, fused=True)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        pg.step(**kw)
    torch.cuda.synchronize()
    for rep in range(3):
        pe.step(**kw)
        graph.replay()
        junk = torch.randn(1 << 20, device=DEV).sum()
        torch.cuda.synchronize()
        pe.check()
        pg.check()
        for i in range(len(shapes)):
            assert torch.equal(We[i], Wg[i]) and torch.equal(Me[i], Mg[i]), f"replay {rep} matrix {i}"
        assert torch.isfinite(junk)
    pe.close()
    pg.close()
    say("  replays equal to the eager fused plan")


@pytest.mark.parametrize("name,nsteps,nesterov", [("illcond768", 1, True), ("aspect3072", 3, False),
                                                  ("aspect3072", 3, True), ("width1024", 3, True)])
def test_fused_matches_staged_on_the_other_workloads(name, nsteps, nesterov):
    """The ill-conditioned, aspect-ratio and width-1024 workloads: the fused
    plan's weights and momentum bitwise equal to the staged plan's after every
    step (the width-1024 set places 144 matrices of three shapes on the XCDs)."""
    say(f"[gpu] fused vs staged, {name}, {nsteps} steps, nesterov={nesterov}")
    wl = inputs.workload(name)
    steps = [inputs.gradients(name, t) for t in range(nsteps)]
    kw = dict(T=5, momentum=wl.momentum, nesterov=nesterov, lr=wl.lr)
    staged = run_plan(wl.shapes, steps, fused=False, **kw)
    fused = run_plan(wl.shapes, steps, fused=True, **kw)
    assert_bitwise(staged, fused, name)
    say(f"  bitwise equal over {nsteps} steps, {len(wl.shapes)} matrices")
