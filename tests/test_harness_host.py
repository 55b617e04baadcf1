"""The GPU tests' closed-form reference for very wide matrices, pinned on the CPU.

``ns_gram_factor`` builds Q with X_T = Q X_0 from the Gram matrix of X_0.  It
must agree with the oracle's step-by-step Newton-Schulz iteration, and with
the SVD closed form, on shapes the oracle runs in milliseconds; a factor
with one step dropped must not.
"""
import numpy as np
import pytest

from muon_harness import A, B, C, O, ns_gram_factor


def x0(rows, cols, seed, rank=None):
    rng = np.random.default_rng(seed)
    X = rng.standard_normal((rows, cols))
    if rank is not None:
        X = rng.standard_normal((rows, rank)) @ rng.standard_normal((rank, cols))
    return O.frobenius_normalise(X)[0]


@pytest.mark.parametrize("rows,cols,rank", [(8, 8, None), (16, 200, None), (33, 517, None), (24, 300, 5),
                                            (1, 64, None)])
def test_gram_factor_equals_the_oracle_iteration(rows, cols, rank):
    X = x0(rows, cols, 11 + rows, rank)
    for T in (1, 5, 9):
        ref = O.newton_schulz(X, A, B, C, T)
        got = ns_gram_factor(X @ X.T, A, B, C, T) @ X
        # rounding in a rank-deficient X's null space grows by a (3.44) per step
        # on both sides: 3.44^9 * 1e-15 is about 7e-11
        assert O.rel_frobenius(got, ref) < 1e-10, (rows, cols, rank, T)


def test_gram_factor_equals_the_svd_closed_form():
    X = x0(20, 90, 3)
    U, S, Vt = np.linalg.svd(X, full_matrices=False)
    s = S.copy()
    a, b, c = O.f32(1.875), O.f32(-1.25), O.f32(0.375)
    for _ in range(7):
        s = a * s + b * s ** 3 + c * s ** 5
    assert O.rel_frobenius(ns_gram_factor(X @ X.T, 1.875, -1.25, 0.375, 7) @ X, (U * s) @ Vt) < 1e-12


def test_a_step_short_fails():
    X = x0(16, 200, 5)
    ref = O.newton_schulz(X, A, B, C, 5)
    assert O.rel_frobenius(ns_gram_factor(X @ X.T, A, B, C, 4) @ X, ref) > 0.05
