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
