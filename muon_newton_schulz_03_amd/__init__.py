"""MI355X (gfx950) Muon optimizer step: HIP kernels behind a C ABI, and a thin binding.

``MuonStep`` runs the whole step (momentum, short-side-first Frobenius
normalisation, quintic Newton-Schulz iterations, weight update) in the HIP
library ``libmuon_mi355x.so``; build it with
``python -m muon_newton_schulz_03_amd.build``.
"""
from .muon import DEFAULT_COEFFS, MuonStep, describe, version  # noqa: F401
