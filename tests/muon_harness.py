"""Shared helpers of the GPU parity tests: run the HIP path and the oracle on one input set."""
from __future__ import annotations

import sys
from dataclasses import dataclass, field
from typing import Dict, List, Optional, Sequence

import numpy as np
import torch

from oracle import muon_oracle as O

A, B, C = 3.4445, -4.7750, 2.0315
TOL_BF16 = 2e-2     # relative Frobenius, bf16 products
TOL_F32 = 1e-4      # relative Frobenius, fp32 path
TOL_MOM = 1e-6      # |M_gpu - M_ref| <= TOL_MOM * max(1, |M_ref|)


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def gpu_available() -> bool:
    return torch.cuda.is_available()


@dataclass
class GpuRun:
    W: List[List[torch.Tensor]] = field(default_factory=list)  # W after each step (CPU copies, sampled)
    M: List[List[torch.Tensor]] = field(default_factory=list)  # momentum after each step (sampled)


def run_gpu(shapes, grads_per_step, *, path="bf16", T=5, mu=0.95, nesterov=True, lr=0.05,
            coeffs=(A, B, C), w0=None, scales=None, x_master_iters=-1, sample=None, keep_steps=None,
            weight_dtype=torch.float32, grads_on_device=False, groups=0, schedule=None):
    """Run the HIP Muon step over the steps' gradients; return sampled W/M after each kept step.

    ``grads_per_step[t]`` is the list of gradients of step t (CPU or device tensors).
    ``sample``: matrix indices to copy back (default all); ``keep_steps``: steps (0-based)
    after which to copy them back (default all).
    """
    from muon_newton_schulz_03_amd import MuonStep

    dev = torch.device("cuda:0")
    n = len(shapes)
    sample = list(range(n)) if sample is None else list(sample)
    keep = set(range(len(grads_per_step))) if keep_steps is None else set(keep_steps)
    if w0 is None:
        W = [torch.zeros(s, dtype=weight_dtype, device=dev) for s in shapes]
    else:
        W = [w.to(dev, weight_dtype).contiguous() for w in w0]
    M = [torch.zeros(s, dtype=torch.float32, device=dev) for s in shapes]
    G = [g.to(dev).clone().contiguous() for g in grads_per_step[0]]  # own buffers
    plan = MuonStep(W, G, M, path=path, x_master_iters=x_master_iters, scales=scales, groups=groups)
    out = GpuRun()
    for t, grads in enumerate(grads_per_step):
        if t > 0:
            for i in range(n):
                G[i].copy_(grads[i].to(dev), non_blocking=False)
        if schedule is not None:
            plan.step(schedule=schedule, momentum=mu, nesterov=nesterov, lr=lr)
        else:
            plan.step(a=coeffs[0], b=coeffs[1], c=coeffs[2], T=T, momentum=mu, nesterov=nesterov, lr=lr)
        if t in keep:
            torch.cuda.synchronize()
            out.W.append([W[i].to("cpu", torch.float64).clone() for i in sample])
            out.M.append([M[i].to("cpu").clone() for i in sample])
        else:
            out.W.append(None)
            out.M.append(None)
    torch.cuda.synchronize()
    plan.close()
    return out


def oracle_steps(w0, grads, *, T=5, mu=0.95, nesterov=True, lr=0.05, coeffs=(A, B, C), scale=1.0,
                 need_ns=None, schedule=None):
    """Oracle over one matrix's step sequence.  ``need_ns``: the steps whose O is
    needed; the others only advance the momentum, and W is then not tracked
    (reported as None)."""
    W = O.as_f64(w0)
    M = np.zeros(W.shape, np.float32)
    res = []
    a, b, c = coeffs
    for t, g in enumerate(grads):
        G = O.as_f64(g)
        if need_ns is None or t in need_ns:
            r = O.muon_step(W if W is not None else np.zeros(G.shape), G, M, a=a, b=b, c=c, T=T, mu=mu,
                            nesterov=nesterov, lr=lr, scale=scale, schedule=schedule)
            M = r.M
            W = r.W if W is not None else None
            res.append(O.StepResult(W, M, r.O, r.nu))
        else:
            M = O.momentum_update(M, G, mu)
            W = None
            res.append(O.StepResult(None, M, None, float("nan")))
    return res


def check_momentum(m_gpu: torch.Tensor, m_ref: np.ndarray, what: str):
    mg = m_gpu.numpy().astype(np.float64)
    mr = m_ref.astype(np.float64)
    err = np.abs(mg - mr) / np.maximum(1.0, np.abs(mr))
    assert err.max() <= TOL_MOM, f"{what}: momentum error {err.max():.3e} > {TOL_MOM}"
    return float(err.max())


def update_from_weights(w_after, w_before, lr, scale=1.0):
    """O recovered from the weight change: (W_before - W_after) / (lr * s)."""
    return (np.asarray(w_before, np.float64) - np.asarray(w_after, np.float64)) / (O.f32(lr) * scale)


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


def ns_gram_factor(A0: np.ndarray, a: float, b: float, c: float, T: int) -> np.ndarray:
    """Q with X_T = Q X_0 after T quintic Newton-Schulz steps, from A0 = X_0 X_0^T alone.

    Each step multiplies X on the left by a polynomial in A_t = X_t X_t^T, and
    every A_t is a polynomial in A0, so all of them share A0's eigenvectors V.
    An eigenvalue s^2 of A0 belongs to a singular value s of X_0, which one step
    maps to s (a + b s^2 + c s^4); hence Q = V diag(prod_t (a + b s_t^2 +
    c s_t^4)) V^T.  This is the SVD closed form the oracle's pins use, reached
    through the m x m Gram matrix, so a reference for X_T costs one pass over
    X_0 whatever its column count.  Coefficients are rounded to fp32 as the
    oracle and the C ABI round them.
    """
    a, b, c = O.f32(a), O.f32(b), O.f32(c)
    lam, V = np.linalg.eigh(np.asarray(A0, np.float64))
    s = np.sqrt(np.clip(lam, 0.0, None))
    g = np.ones_like(s)
    for _ in range(T):
        p = a + b * s * s + c * s ** 4
        g *= p
        s = s * p
    return (V * g) @ V.T


@dataclass
class StreamResult:
    worst: Dict[int, float] = field(default_factory=dict)       # worst rel err of O per compared matrix
    w_final: Dict[int, np.ndarray] = field(default_factory=dict)  # tracked: GPU weights after the last step
    w_ref: Dict[int, np.ndarray] = field(default_factory=dict)    # tracked: oracle weights after the last step
    compared: int = 0                                             # (matrix, step) pairs compared


def stream_parity(shapes, grads_at, nsteps, *, check, track=(), path="bf16", T=5, mu=0.95, nesterov=True,
                  lr=0.05, coeffs=(A, B, C), groups=0, tol=None) -> StreamResult:
    """Run ``nsteps`` HIP steps over all ``shapes`` and compare as they go.

    ``grads_at(t)`` returns step t's gradients (one tensor per matrix).  After
    step t the matrices ``check(t)`` are compared with the oracle: O recovered
    from the step's weight change (rel. Frobenius <= tol) and the momentum
    buffer elementwise.  The oracle keeps state only for the matrices that are
    ever checked or tracked: it advances their momentum every step and runs
    the Newton-Schulz iteration at the steps that compare them; for the
    ``track`` matrices it runs every step and keeps their weights, which are
    returned with the GPU's after the last step.  Weights start at zero.
    """
    from muon_newton_schulz_03_amd import MuonStep

    tol = tol if tol is not None else (TOL_F32 if path == "f32" else TOL_BF16)
    dev = torch.device("cuda:0")
    n = len(shapes)
    track = set(track)
    union = sorted(set().union(*[set(check(t)) for t in range(nsteps)]) | track)
    W = [torch.zeros(s, dtype=torch.float32, device=dev) for s in shapes]
    M = [torch.zeros(s, dtype=torch.float32, device=dev) for s in shapes]
    g0 = grads_at(0)
    G = [g.to(dev).clone().contiguous() for g in g0]
    plan = MuonStep(W, G, M, path=path, groups=groups)
    m_ref = {i: np.zeros(shapes[i], np.float32) for i in union}
    w_ref = {i: np.zeros(shapes[i], np.float64) for i in track}
    w_prev = {i: np.zeros(shapes[i], np.float32) for i in union}
    res = StreamResult()
    a, b, c = coeffs
    for t in range(nsteps):
        grads = g0 if t == 0 else grads_at(t)
        if t > 0:
            for i in range(n):
                G[i].copy_(grads[i].to(dev))
        plan.step(a=a, b=b, c=c, T=T, momentum=mu, nesterov=nesterov, lr=lr)
        torch.cuda.synchronize()
        want = set(check(t))
        for i in union:
            g = O.as_f64(grads[i].cpu())
            w_now = W[i].cpu().numpy()
            if i in want or i in track:
                r = O.muon_step(w_ref[i] if i in track else np.zeros(shapes[i]), g, m_ref[i], a=a, b=b, c=c,
                                T=T, mu=mu, nesterov=nesterov, lr=lr)
                m_ref[i] = r.M
                if i in track:
                    w_ref[i] = r.W
                if i in want:
                    og = update_from_weights(w_now, w_prev[i], lr)
                    e = O.rel_frobenius(og, r.O)
                    res.worst[i] = max(res.worst.get(i, 0.0), e)
                    res.compared += 1
                    assert e <= tol, f"matrix {i} {shapes[i]} step {t}: rel err {e:.3e} > {tol}"
                    check_momentum(M[i].cpu(), r.M, f"matrix {i} step {t}")
            else:
                m_ref[i] = O.momentum_update(m_ref[i], g, mu)
            w_prev[i] = w_now
        say(f"  step {t + 1}/{nsteps}: {len(want)} matrices compared, worst so far "
            f"{max(res.worst.values()) if res.worst else 0.0:.3e}")
    for i in track:
        res.w_final[i] = W[i].cpu().numpy().astype(np.float64)
        res.w_ref[i] = w_ref[i]
    plan.close()
    return res
