"""muon_step_scratch (the allocation-free step) against muon_init + muon_step.

Both run the same kernels in the same order on one stream, so the weights and
momentum buffers they produce must agree bitwise; two calls in a row, the
second on a smaller set, show that what the first call left in the shared
static array does not leak into the second.  A set whose working memory
exceeds the array is refused before anything is enqueued.
"""
import pytest
import torch

from muon_harness import say
from muon_newton_schulz_03_amd import MuonStep, inputs
from muon_newton_schulz_03_amd._lib import MUON_E_WORKSPACE, MuonError
from muon_newton_schulz_03_amd.muon import step_scratch

pytestmark = pytest.mark.gpu

KW = dict(T=5, momentum=0.95, nesterov=True, lr=0.1)


def tensors(shapes, seed, dev, w_dtype=torch.float32):
    W = [inputs.custom_gradient(r, c, seed + 50 + i, torch.float32, std=0.1).to(dev, w_dtype) for i, (r, c) in
         enumerate(shapes)]
    G = [inputs.custom_gradient(r, c, seed + i, std=0.02).to(dev) for i, (r, c) in enumerate(shapes)]
    M = [inputs.custom_gradient(r, c, seed + 100 + i, torch.float32, std=0.01).to(dev) for i, (r, c) in
         enumerate(shapes)]
    return W, G, M


def planned_step(W, G, M, path):
    p = MuonStep(W, G, M, path=path, groups=1)
    p.step(**KW)
    torch.cuda.synchronize()
    p.close()


@pytest.mark.parametrize("path", ["bf16", "f32"])
def test_scratch_step_equals_planned_step(path):
    dev = "cuda:0"
    calls = [
        [(256, 384), (384, 256), (768, 768), (100, 37), (768, 3072)],  # larger first
        [(130, 130), (64, 200)],                                        # then smaller
    ]
    for k, shapes in enumerate(calls):
        say(f"[gpu] scratch step path={path} call {k + 1}: {shapes}")
        W1, G1, M1 = tensors(shapes, 300 + 10 * k, dev)
        W2, G2, M2 = [w.clone() for w in W1], [g.clone() for g in G1], [m.clone() for m in M1]
        planned_step(W1, G1, M1, path)
        step_scratch(W2, G2, M2, path=path, **KW)
        torch.cuda.synchronize()
        for i in range(len(shapes)):
            assert torch.equal(W1[i], W2[i]), f"call {k + 1} matrix {i} {shapes[i]}: weights differ"
            assert torch.equal(M1[i], M2[i]), f"call {k + 1} matrix {i} {shapes[i]}: momentum differs"
            assert torch.isfinite(W2[i]).all()
        assert any(not torch.equal(w, w0) for w, w0 in zip(W2, tensors(shapes, 300 + 10 * k, dev)[0]))


def test_scratch_step_refuses_sets_beyond_its_array():
    dev = "cuda:0"
    shapes = [(768, 3072)] * 6  # working memory ~85 MiB > 64 MiB
    W, G, M = tensors(shapes, 900, dev)
    before = [w.clone() for w in W]
    with pytest.raises(MuonError, match="scratch") as err:
        step_scratch(W, G, M, **KW)
    assert err.value.code == MUON_E_WORKSPACE
    torch.cuda.synchronize()
    assert all(torch.equal(w, b) for w, b in zip(W, before))


def test_scratch_steps_back_to_back():
    """Two calls enqueued without a host synchronisation in between (the second
    smaller): each must still read its own tables."""
    dev = "cuda:0"
    first, second = [(256, 384), (768, 768), (384, 256)], [(130, 130)]
    sets = [tensors(first, 400, dev), tensors(second, 410, dev)]
    refs = [[[t.clone() for t in part] for part in s] for s in sets]
    for W, G, M in refs:
        planned_step(W, G, M, "bf16")
    for W, G, M in sets:
        step_scratch(W, G, M, **KW)
    torch.cuda.synchronize()
    for (W, _, M), (Wr, _, Mr) in zip(sets, refs):
        for i in range(len(W)):
            assert torch.equal(W[i], Wr[i]) and torch.equal(M[i], Mr[i]), i
