"""Parity at the largest matrices muon_init accepts (needs an MI355X).

A side may hold up to 2^20 elements, and each buffer of a matrix (weights,
momentum, and the padded X of the products) must stay below 2 GiB, since the
kernels address a matrix with 32-bit byte offsets.  These tests run one step
on matrices at those bounds:
  * the longest side, 2^20, on the bf16 products (128 rows, and its
    transpose) and on the fp32 products (100 rows, 2^20 - 1 columns), against
    the oracle step for step;
  * 512 x 1,048,447, whose fp32 weights and momentum take 2^31 - 258 KiB each:
    momentum against the oracle's momentum update element by element, and
    the whole update against the exact result of the iteration, computed
    from the 512 x 512 Gram matrix (``ns_gram_factor``, pinned to the oracle
    on the CPU), since the oracle's own iteration would take minutes there.
"""
import math

import numpy as np
import pytest
import torch

from muon_harness import A, B, C, TOL_BF16, O, check_momentum, compare_run, ns_gram_factor, run_gpu, say
from muon_newton_schulz_03_amd import inputs

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
LONG = 1 << 20


def padded_bytes(rows, cols, elem=4):
    m, n = min(rows, cols), max(rows, cols)
    return (-(-m // 256) * 256) * (-(-n // 128) * 128) * elem


def test_longest_side():
    shapes = [(128, LONG), (LONG, 128), (100, LONG - 1)]
    say(f"[gpu] longest side: {shapes}")
    steps = [[inputs.custom_gradient(r, c, 8800 + i, std=0.02) for i, (r, c) in enumerate(shapes)]]
    w0 = inputs.weights(shapes, seed=88)
    gpu = run_gpu(shapes, steps, path="bf16", lr=0.05, w0=w0)
    say("  step done; oracle")
    worst = compare_run(shapes, steps, gpu, path="bf16", lr=0.05, mu=0.95, nesterov=True, w0=w0)
    say(f"  worst rel err {worst:.3e}")


def test_two_gib_buffers():
    rows, cols = 512, 1048447
    lim = 1 << 31
    assert lim - (1 << 20) < rows * cols * 4 < lim and padded_bytes(rows, cols) < lim
    mu, lr, T = 0.95, 0.05, 5
    say(f"[gpu] 2 GiB buffers: {rows} x {cols}, {rows * cols * 4} bytes of fp32 weights and momentum")
    g = inputs.custom_gradient(rows, cols, 8900, std=0.02)
    w0 = inputs.weights([(rows, cols)], seed=89)[0]
    m0 = inputs.weights([(rows, cols)], seed=90, std=0.02)[0]  # a momentum buffer from earlier steps
    from muon_newton_schulz_03_amd import MuonStep
    W, M, G = w0.to(DEV), m0.to(DEV), g.to(DEV)
    plan = MuonStep([W], [G], [M])
    plan.step(a=A, b=B, c=C, T=T, momentum=mu, nesterov=True, lr=lr)
    torch.cuda.synchronize()
    plan.close()
    w1, m1 = W.cpu(), M.cpu()
    del W, M, G
    torch.cuda.empty_cache()
    say("  step done; reference")

    chunk = 1 << 17
    spans = [(j, min(cols, j + chunk)) for j in range(0, cols, chunk)]

    # U = G + mu M' per column block (the oracle's momentum update and Nesterov
    # blend), kept for the three passes: 4.3 GB of fp64
    us = []
    ss = 0.0
    for j0, j1 in spans:
        gj = O.as_f64(g[:, j0:j1])
        mj = O.momentum_update(m0[:, j0:j1].numpy(), gj, mu)
        check_momentum(m1[:, j0:j1], mj, f"columns {j0}..{j1}")
        us.append(O.nesterov_blend(gj, mj, mu, True))
        ss += float(np.sum(us[-1] * us[-1]))
    inv = 1.0 / (math.sqrt(ss) + O.EPS)
    A0 = np.zeros((rows, rows))
    for u in us:
        A0 += u @ u.T
    Q = ns_gram_factor(A0 * (inv * inv), A, B, C, T)
    err2 = ref2 = 0.0
    blocks, colerr = [], []
    rowd2, rowr2 = np.zeros(rows), np.zeros(rows)
    for (j0, j1), u in zip(spans, us):
        ref = Q @ (u * inv)
        got = (O.as_f64(w0[:, j0:j1]) - O.as_f64(w1[:, j0:j1])) / O.f32(lr)
        d2 = np.sum((got - ref) ** 2, axis=0)
        r2 = np.sum(ref * ref, axis=0)
        err2, ref2 = err2 + float(d2.sum()), ref2 + float(r2.sum())
        blocks.append(math.sqrt(d2.sum() / r2.sum()))
        colerr.append(np.sqrt(d2 / r2))
        rowd2 += np.sum((got - ref) ** 2, axis=1)
        rowr2 += np.sum(ref * ref, axis=1)
    rel = math.sqrt(err2 / ref2)
    ce = np.concatenate(colerr)
    worst = np.argsort(ce)[-5:][::-1]
    say(f"  rel err {rel:.3e}; per column block " + " ".join(f"{e:.2e}" for e in blocks))
    say(f"  per column: median {np.median(ce):.3e}, p99.9 {np.percentile(ce, 99.9):.3e}, worst "
        + ", ".join(f"{int(j)}: {ce[j]:.2e}" for j in worst))
    re = np.sqrt(rowd2 / rowr2)
    say(f"  per row: median {np.median(re):.3e}, worst " + ", ".join(f"{int(i)}: {re[i]:.2e}" for i in np.argsort(re)[-5:][::-1]))
    assert rel <= TOL_BF16, f"rel err {rel:.3e}"
    for (j0, j1), e in zip(spans, blocks):
        assert e <= TOL_BF16, f"columns {j0}..{j1}: rel err {e:.3e}"
