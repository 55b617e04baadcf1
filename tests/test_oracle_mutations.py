"""Planted mistakes in the oracle (on the CPU) must fail its pins.

Each mutant replaces one oracle function with a plausibly wrong version; the
test asserts that at least one pin check then fails.  This shows the pins
are strong enough to catch the mistakes they are meant to catch.
"""
import numpy as np
import pytest

from oracle import muon_oracle as O
from test_oracle_pins import A, B, C, ns_via_svd, p_iter, rng


def ns_transposed_gram(X0, a, b, c, T):
    a, b, c = O.f32(a), O.f32(b), O.f32(c)
    X = X0
    for _ in range(T):
        A_ = X.T @ X                      # wrong Gram side, applied on the left
        X = a * X + (b * A_ + c * A_ @ A_) @ X
    return X


def ns_dropped_quintic(X0, a, b, c, T):
    a, b, c = O.f32(a), O.f32(b), O.f32(c)
    X = X0
    for _ in range(T):
        A_ = X @ X.T
        X = a * X + (b * A_) @ X          # c A^2 term dropped
    return X


def ns_sign(X0, a, b, c, T):
    return O.newton_schulz(X0, a, -b, c, T)


def ns_one_short(X0, a, b, c, T):
    return O.newton_schulz(X0, a, b, c, max(T - 1, 0))


def ns_swapped_ab(X0, a, b, c, T):
    return O.newton_schulz(X0, b, a, c, T)


def pin_closed_form(ns):
    for shape in [(33, 33), (24, 40)]:
        G = rng(21).standard_normal(shape)
        X0, _ = O.frobenius_normalise(G)
        try:
            out = ns(X0, A, B, C, 5)
        except ValueError:  # shape mismatch: the pin fails loudly
            return False
        if O.rel_frobenius(out, ns_via_svd(X0, A, B, C, 5)) > 1e-10:
            return False
    return True


def pin_identity_block(ns):
    e = np.hstack([np.eye(4), np.zeros((4, 4))])
    X0 = e / (2.0 + O.EPS)
    try:
        ns(X0, A, B, C, 5)
    except ValueError:
        return False
    return O.rel_frobenius(ns(X0, A, B, C, 5), p_iter(1 / (2 + O.EPS), 5) * e) < 1e-12


@pytest.mark.parametrize("mutant", [ns_transposed_gram, ns_dropped_quintic, ns_sign,
                                    ns_one_short, ns_swapped_ab])
def test_mutants_fail_a_pin(mutant):
    assert pin_closed_form(O.newton_schulz) and pin_identity_block(O.newton_schulz)
    assert not (pin_closed_form(mutant) and pin_identity_block(mutant))


def test_momentum_mutants_fail_hand_example():
    g1 = np.arange(32, dtype=np.float64).reshape(4, 8) - 11.0
    g2 = (np.arange(32, dtype=np.float64).reshape(4, 8) % 5) * 3.0 - 4.0

    def ema(M, G, mu):  # EMA form instead of the SGD form
        return ((O.f32(mu) * M + (1 - O.f32(mu)) * G)).astype(np.float32)

    def swapped(M, G, mu):
        return (O.f32(mu) * G + M).astype(np.float32)

    for mom in (O.momentum_update, ema, swapped):
        m2 = mom(mom(np.zeros((4, 8), np.float32), g1, 0.5), g2, 0.5)
        ok = np.array_equal(m2, 0.5 * g1 + g2)
        assert ok == (mom is O.momentum_update)


def test_schedule_mutants_fail_the_closed_form():
    from test_oracle_pins import SCHEDULE, schedule_via_svd

    def reversed_order(X0, schedule):
        return O.newton_schulz_schedule(X0, list(schedule)[::-1])

    def first_triple_only(X0, schedule):
        return O.newton_schulz(X0, *schedule[0], len(schedule))

    def pin(ns):
        G = rng(41).standard_normal((30, 50))
        X0, _ = O.frobenius_normalise(G)
        return O.rel_frobenius(ns(X0, SCHEDULE), schedule_via_svd(X0, SCHEDULE)) < 1e-10

    assert pin(O.newton_schulz_schedule)
    assert not pin(reversed_order)
    assert not pin(first_triple_only)
