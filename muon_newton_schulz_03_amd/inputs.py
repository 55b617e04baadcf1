"""Seeded synthetic inputs for the Muon step (no Muon arithmetic lives here).

Both sides of every comparison draw their inputs from this module: the HIP
path and the fp64 oracle receive the very same tensors.  Nothing in here
computes any part of the update (momentum, normalisation, Newton-Schulz or
the weight step); it only draws random numbers, shapes them like the hidden
matrices of the models named on the pages, and rounds them to the storage
dtype the workload prescribes.

Workloads (shapes and value distributions):

* ``single768``: one 768x768 fp32 gradient with i.i.d. N(0,1) entries
  (fp32 path).
* ``gpt2_small``: the hidden matrices of the 12-layer, width-768 GPT-2 small
  model whose training the pages time (speedrun overview page, "Context"):
  per layer four 768x768 attention matrices, one 768x3072 MLP-in and one
  3072x768 MLP-out, 72 in all; bf16 gradients of 0.02*N(0,1).
* ``illcond768``: 24 matrices of 768x768 built as U*diag(s)*V^T with Haar
  orthogonal U, V and singular values log-uniform in [1e-4, 1], plus
  1e-6*N(0,1) noise, stored bf16.
* ``aspect3072``: 48 matrices alternating 3072x768 and 768x3072, bf16
  0.02*N(0,1) with round(5% of rows) rows (seeded choice) scaled by 50.
* ``width1024``: 24 layers of {4 x 1024x1024, 1024x4096, 4096x1024},
  144 matrices, bf16 0.02*N(0,1).

Seeding: every gradient matrix has its own seed,
``base(workload) + 100_000*run + 1_000*step + index``, drawn with a
``torch.Generator`` on the requested device.  The CPU and GPU generators
produce different streams, so a comparison always hands the one tensor it
drew to both sides.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import List, Sequence, Tuple

import torch

WORKLOADS = ("single768", "gpt2_small", "illcond768", "aspect3072", "width1024")

_SEED_BASE = {
    "single768": 0,
    "gpt2_small": 2_000_000,
    "illcond768": 3_000_000,
    "aspect3072": 4_000_000,
    "width1024": 5_000_000,
    "custom": 7_000_000,
}


@dataclass
class Workload:
    """Shapes, gradient dtype and hyper-parameters of one synthetic workload."""

    name: str
    shapes: List[Tuple[int, int]]
    grad_dtype: torch.dtype
    path: str  # "bf16" or "f32": the arithmetic the Newton-Schulz products use
    steps: int
    momentum: float = 0.95
    nesterov: bool = True
    lr: float = 0.05
    T: int = 5
    coeffs: Tuple[float, float, float] = (3.4445, -4.7750, 2.0315)
    extra: dict = field(default_factory=dict)

    @property
    def params(self) -> int:
        return sum(r * c for r, c in self.shapes)


def gpt2_hidden_shapes(layers: int = 12, width: int = 768) -> List[Tuple[int, int]]:
    """Per layer: 4 square attention matrices, MLP-in (w x 4w), MLP-out (4w x w)."""
    shapes: List[Tuple[int, int]] = []
    for _ in range(layers):
        shapes += [(width, width)] * 4
        shapes.append((width, 4 * width))
        shapes.append((4 * width, width))
    return shapes


def workload(name: str) -> Workload:
    if name == "single768":
        return Workload(name, [(768, 768)], torch.float32, "f32", steps=1, lr=1.0)
    if name == "gpt2_small":
        return Workload(name, gpt2_hidden_shapes(12, 768), torch.bfloat16, "bf16", steps=10)
    if name == "illcond768":
        return Workload(name, [(768, 768)] * 24, torch.bfloat16, "bf16", steps=1, lr=1.0)
    if name == "aspect3072":
        shapes = [(3072, 768) if i % 2 == 0 else (768, 3072) for i in range(48)]
        return Workload(name, shapes, torch.bfloat16, "bf16", steps=3, lr=1.0)
    if name == "width1024":
        return Workload(name, gpt2_hidden_shapes(24, 1024), torch.bfloat16, "bf16", steps=50)
    raise KeyError(name)


def seed_for(name: str, step: int, index: int, run: int = 0) -> int:
    return _SEED_BASE[name] + 100_000 * run + 1_000 * step + index


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def gaussian(shape: Sequence[int], std: float, seed: int, device="cpu",
             dtype: torch.dtype = torch.bfloat16) -> torch.Tensor:
    """std*N(0,1) drawn in fp32, then rounded (RNE) to ``dtype``."""
    x = torch.randn(tuple(shape), generator=_gen(seed, device), device=device,
                    dtype=torch.float32)
    if std != 1.0:
        x.mul_(std)
    return x.to(dtype)


def heavy_rows_gaussian(shape: Sequence[int], std: float, frac: float, factor: float,
                        seed: int, device="cpu", dtype=torch.bfloat16) -> torch.Tensor:
    """std*N(0,1) with round(frac*rows) seeded rows multiplied by ``factor``."""
    rows = shape[0]
    g = _gen(seed, device)
    x = torch.randn(tuple(shape), generator=g, device=device, dtype=torch.float32)
    x.mul_(std)
    k = int(round(frac * rows))
    perm = torch.randperm(rows, generator=g, device=device)[:k]
    x[perm] *= factor
    return x.to(dtype)


def haar_orthogonal(n: int, gen: torch.Generator) -> torch.Tensor:
    """Haar orthogonal n x n (fp64, CPU): QR of a Gaussian, columns sign-fixed by diag(R)."""
    z = torch.randn(n, n, generator=gen, dtype=torch.float64)
    q, r = torch.linalg.qr(z)
    return q * torch.sign(torch.diagonal(r)).unsqueeze(0)


def illconditioned(n: int, seed: int, smin: float = 1e-4, smax: float = 1.0,
                   noise: float = 1e-6, dtype=torch.bfloat16) -> torch.Tensor:
    """U diag(s) V^T + noise*N(0,1), s log-uniform in [smin, smax], built on the CPU."""
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    u = haar_orthogonal(n, g)
    v = haar_orthogonal(n, g)
    lo, hi = math.log(smin), math.log(smax)
    s = torch.exp(lo + (hi - lo) * torch.rand(n, generator=g, dtype=torch.float64))
    x = (u * s.unsqueeze(0)) @ v.T
    x = x + noise * torch.randn(n, n, generator=g, dtype=torch.float64)
    return x.to(dtype)


def gradients(name: str, step: int, run: int = 0, device="cpu",
              indices: Sequence[int] | None = None) -> List[torch.Tensor]:
    """The gradients of ``step`` (0-based) for every matrix of the workload.

    ``indices`` restricts the draw to some matrices; each matrix has its own
    seed, so a subset is bit-identical to the same entries of the full set.
    """
    wl = workload(name)
    idx = range(len(wl.shapes)) if indices is None else indices
    out = []
    for i in idx:
        shape = wl.shapes[i]
        seed = seed_for(name, step, i, run)
        if name == "single768":
            out.append(gaussian(shape, 1.0, seed, device, torch.float32))
        elif name == "illcond768":
            out.append(illconditioned(shape[0], seed).to(device))
        elif name == "aspect3072":
            out.append(heavy_rows_gaussian(shape, 0.02, 0.05, 50.0, seed, device))
        else:
            out.append(gaussian(shape, 0.02, seed, device, torch.bfloat16))
    return out


def orthonormal_rows(rows: int, cols: int, seed: int, scale: float = 0.02,
                     dtype=torch.bfloat16) -> torch.Tensor:
    """scale * Q with orthonormal rows or columns (QR of a seeded Gaussian, built
    in fp64 on the CPU), rows x cols: every singular value equal to ``scale``
    before the rounding to ``dtype``.  A flat spectrum is the degenerate case
    of the iteration in which all singular values take the same path."""
    m, n = min(rows, cols), max(rows, cols)
    g = _gen(_SEED_BASE["custom"] + 7919 * seed, "cpu")
    q, r = torch.linalg.qr(torch.randn(n, m, generator=g, dtype=torch.float64))
    q = q * torch.sign(torch.diagonal(r)).unsqueeze(0)  # n x m, orthonormal columns
    x = q.T if rows <= cols else q
    return (scale * x).contiguous().to(dtype)


def custom_gradient(rows: int, cols: int, seed: int, dtype=torch.bfloat16, std: float = 1.0,
                    device="cpu") -> torch.Tensor:
    """One std*N(0,1) matrix of an arbitrary shape (ragged and edge-case tests)."""
    return gaussian((rows, cols), std, _SEED_BASE["custom"] + seed, device, dtype)


def weights(shapes: Sequence[Tuple[int, int]], seed: int | None, device="cpu",
            dtype=torch.float32, std: float = 0.02) -> List[torch.Tensor]:
    """Initial weights: zeros when ``seed`` is None, else std*N(0,1)."""
    if seed is None:
        return [torch.zeros(s, dtype=dtype, device=device) for s in shapes]
    return [gaussian(s, std, seed + i, device, dtype) for i, s in enumerate(shapes)]
