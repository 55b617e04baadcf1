"""The seeded workload generators: shapes, dtypes, distributions, determinism."""
import math

import numpy as np
import pytest
import torch

from muon_newton_schulz_03_amd import inputs


def test_workload_shapes():
    g = inputs.workload("gpt2_small")
    assert len(g.shapes) == 72 and g.params == 84_934_656
    assert g.shapes[:6] == [(768, 768)] * 4 + [(768, 3072), (3072, 768)]
    w = inputs.workload("width1024")
    assert len(w.shapes) == 144 and w.params == 301_989_888
    a = inputs.workload("aspect3072")
    assert len(a.shapes) == 48 and a.shapes[0] == (3072, 768) and a.shapes[1] == (768, 3072)
    assert inputs.workload("illcond768").shapes == [(768, 768)] * 24
    s = inputs.workload("single768")
    assert s.shapes == [(768, 768)] and s.grad_dtype == torch.float32 and s.path == "f32"


def test_gradients_are_seeded_per_matrix():
    full = inputs.gradients("gpt2_small", step=3, indices=[0, 4, 5])
    again = inputs.gradients("gpt2_small", step=3, indices=[5])
    assert torch.equal(full[2], again[0])
    other = inputs.gradients("gpt2_small", step=4, indices=[5])
    assert not torch.equal(other[0], again[0])
    assert full[0].dtype == torch.bfloat16 and full[1].shape == (768, 3072)
    x = full[1].float()
    assert abs(x.std().item() - 0.02) < 5e-4 and abs(x.mean().item()) < 2e-4


def test_heavy_rows():
    g = inputs.gradients("aspect3072", step=0, indices=[0, 1])
    for t in g:
        rows = t.shape[0]
        norms = t.float().norm(dim=1)
        big = (norms > 10 * norms.median()).sum().item()
        assert big == round(0.05 * rows)


def test_illconditioned_spectrum():
    x = inputs.illconditioned(96, seed=1).double().numpy()
    sv = np.linalg.svd(x, compute_uv=False)
    assert sv.max() <= 1.0 + 1e-2 and sv.max() > 0.5
    assert sv.min() < 1e-3
    # log-uniform singular values: their logs spread over [ln 1e-4, 0]
    logs = np.log(sv[sv > 1e-5])
    assert logs.min() < math.log(1e-3)


def test_single768_fp32_normal():
    (g,) = inputs.gradients("single768", step=0)
    assert g.dtype == torch.float32 and g.shape == (768, 768)
    assert abs(g.std().item() - 1.0) < 0.01


@pytest.mark.parametrize("seed", [None, 5])
def test_weights(seed):
    w = inputs.weights([(3, 4), (5, 2)], seed)
    assert [t.shape for t in w] == [(3, 4), (5, 2)]
    assert (seed is None) == all(not t.any() for t in w)


def test_orthonormal_rows_have_a_flat_spectrum():
    for shape in [(64, 300), (300, 64), (50, 50)]:
        x = inputs.orthonormal_rows(*shape, seed=3, scale=0.5)
        assert x.shape == shape and x.dtype == torch.bfloat16
        sv = torch.linalg.svdvals(x.double())
        assert float(sv.max() / sv.min()) < 1.02  # bf16 rounding only
        assert abs(float(sv.mean()) - 0.5) < 5e-3
    assert torch.equal(inputs.orthonormal_rows(64, 300, 3), inputs.orthonormal_rows(64, 300, 3))
    assert not torch.equal(inputs.orthonormal_rows(64, 300, 3), inputs.orthonormal_rows(64, 300, 4))
