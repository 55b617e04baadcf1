"""Pins of the fp64 oracle against facts fixed outside the oracle itself.

Each pin uses a route the oracle does not take: the SVD closed form of the
polynomial iteration, exact rational arithmetic, textbook special cases,
invariances, the polar factor from a library SVD, and values the pages print.
A dropped term, a wrong sign, a transposed operand or a wrong coefficient in
the oracle fails at least one of them.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

from golden_io import read_golden
from oracle import muon_oracle as O
from muon_newton_schulz_03_amd import inputs

A, B, C = 3.4445, -4.7750, 2.0315
A32, B32, C32 = (O.f32(v) for v in (A, B, C))


def p_scalar(s, a=A32, b=B32, c=C32):
    return a * s + b * s ** 3 + c * s ** 5


def p_iter(s, T, a=A32, b=B32, c=C32):
    for _ in range(T):
        s = p_scalar(s, a, b, c)
    return s


def p_iter_exact(s, T, coeffs):
    a, b, c = (Fraction(x) for x in coeffs)
    s = Fraction(s)
    for _ in range(T):
        s = a * s + b * s ** 3 + c * s ** 5
    return s


def ns_via_svd(X0, a, b, c, T):
    """Closed form: if X0 = U S V^T then each step maps S -> aS + bS^3 + cS^5."""
    U, S, Vt = np.linalg.svd(X0, full_matrices=False)
    S = p_iter(S, T, O.f32(a), O.f32(b), O.f32(c))
    return (U * S) @ Vt


def rng(seed):
    return np.random.default_rng(seed)


# --- P1: whole iteration against the SVD closed form ------------------------

@pytest.mark.parametrize("shape", [(96, 96), (48, 160), (160, 48), (7, 13)])
def test_ns_matches_svd_closed_form(shape):
    G = rng(1).standard_normal(shape)
    X, transposed = O.to_short_side_first(G)
    X0, _ = O.frobenius_normalise(X)
    got = O.newton_schulz(X0, A, B, C, 5)
    ref = ns_via_svd(X0, A, B, C, 5)
    assert O.rel_frobenius(got, ref) < 1e-13
    # through the full orthogonalise (short side first, then back)
    Ofull, _ = O.orthogonalise(G, A, B, C, 5)
    ref_full = ref.T if transposed else ref
    assert Ofull.shape == G.shape
    assert O.rel_frobenius(Ofull, ref_full) < 1e-13


def test_ns_closed_form_other_T_and_coeffs():
    G = rng(2).standard_normal((40, 72))
    X0, _ = O.frobenius_normalise(G)
    for (a, b, c), T in [((A, B, C), 1), ((A, B, C), 3), ((1.5, -0.5, 0.0), 7),
                         ((15 / 8, -10 / 8, 3 / 8), 4), ((2.0, 0.0, -1.0), 2)]:
        got = O.newton_schulz(X0, a, b, c, T)
        assert O.rel_frobenius(got, ns_via_svd(X0, a, b, c, T)) < 1e-13


# --- P2: the scalar map on 1x1 inputs, in exact rational arithmetic ---------

def test_scalar_map_exact():
    coeffs32 = (A32, B32, C32)
    for s, T in [(1.0, 1), (1.0, 5), (0.5, 5), (0.25, 3), (768 ** -0.5, 5), (1024 ** -0.5, 5)]:
        got = O.newton_schulz(np.array([[s]]), A, B, C, T)[0, 0]
        assert abs(got - float(p_iter_exact(s, T, coeffs32))) < 1e-12


def test_scalar_map_textbook_values():
    # with the decimal coefficients: p(1) = a + b + c = 0.7010 exactly
    assert p_iter_exact(1, 1, ("3.4445", "-4.7750", "2.0315")) == Fraction("0.7010")
    # fp32 rounding of the coefficients moves p(1) by < 1e-6
    got = O.newton_schulz(np.array([[1.0]]), A, B, C, 1)[0, 0]
    assert abs(got - 0.7010) < 1e-6
    # iteration zero is the identity
    assert O.newton_schulz(np.array([[0.3]]), A, B, C, 0)[0, 0] == 0.3


# --- P3: special inputs with closed-form results ----------------------------

def test_orthogonal_input():
    n = 96
    Q, _ = np.linalg.qr(rng(3).standard_normal((n, n)))
    out, nu = O.orthogonalise(Q, A, B, C, 5)
    sigma = 1.0 / (np.sqrt(n) + O.EPS)
    assert abs(nu - np.sqrt(n)) < 1e-12
    assert O.rel_frobenius(out, p_iter(sigma, 5) * Q) < 1e-12


def test_rank_one_input():
    r = rng(4)
    u, v = r.standard_normal(24), r.standard_normal(40)
    G = np.outer(u, v)
    nrm = np.linalg.norm(u) * np.linalg.norm(v)
    out, _ = O.orthogonalise(G, A, B, C, 5)
    sigma = nrm / (nrm + O.EPS)
    assert O.rel_frobenius(out, p_iter(sigma, 5) * G / nrm) < 1e-12


@pytest.mark.parametrize("transpose", [False, True])
def test_identity_block_4x8(transpose):
    G = np.hstack([np.eye(4), np.zeros((4, 4))])
    if transpose:
        G = G.T  # 8x4: exercises the short-side-first transpose
    out, nu = O.orthogonalise(G, A, B, C, 5)
    assert nu == 2.0
    sigma = 1.0 / (2.0 + O.EPS)
    assert O.rel_frobenius(out, p_iter(sigma, 5) * G) < 1e-13
    # with the decimal coefficients p^5(1/2) = 0.76543853045...
    assert abs(float(p_iter_exact(0.5, 5, ("3.4445", "-4.7750", "2.0315"))) - 0.765438530454) < 1e-12


def test_zero_gradient_gives_zero_update():
    out, nu = O.orthogonalise(np.zeros((5, 9)), A, B, C, 5)
    assert nu == 0.0 and not np.any(out)
    r = O.muon_step(np.ones((5, 9)), np.zeros((5, 9)), np.zeros((5, 9), np.float32),
                    a=A, b=B, c=C, T=5, mu=0.95, nesterov=True, lr=0.1)
    assert np.array_equal(r.W, np.ones((5, 9)))


# --- P4: invariances ---------------------------------------------------------

def test_invariances():
    r = rng(5)
    G = r.standard_normal((30, 50))
    base, _ = O.orthogonalise(G, A, B, C, 5)
    t, _ = O.orthogonalise(G.T, A, B, C, 5)
    assert O.rel_frobenius(t, base.T) == 0.0            # transpose rule
    neg, _ = O.orthogonalise(-G, A, B, C, 5)
    assert O.rel_frobenius(neg, -base) < 1e-15           # odd map
    sc, _ = O.orthogonalise(1e3 * G, A, B, C, 5)
    assert O.rel_frobenius(sc, base) < 1e-7              # scale (up to eps)
    Q1, _ = np.linalg.qr(r.standard_normal((30, 30)))
    Q2, _ = np.linalg.qr(r.standard_normal((50, 50)))
    eq, _ = O.orthogonalise(Q1 @ G @ Q2, A, B, C, 5)
    assert O.rel_frobenius(eq, Q1 @ base @ Q2) < 1e-12   # orthogonal equivariance


# --- P5: convergent coefficients reach the polar factor ---------------------

def polar(G):
    U, _, Vt = np.linalg.svd(G, full_matrices=False)
    return U @ Vt


def well_conditioned(rows, cols, cond, seed):
    r = rng(seed)
    U, _ = np.linalg.qr(r.standard_normal((rows, min(rows, cols))))
    V, _ = np.linalg.qr(r.standard_normal((cols, min(rows, cols))))
    s = np.linspace(1.0, 1.0 / cond, min(rows, cols))
    return (U * s) @ V.T


@pytest.mark.parametrize("coeffs,T", [((1.5, -0.5, 0.0), 15), ((15 / 8, -10 / 8, 3 / 8), 10)])
@pytest.mark.parametrize("shape", [(32, 64), (64, 32)])
def test_convergent_coefficients_reach_polar(coeffs, T, shape):
    G = well_conditioned(*shape, cond=5.0, seed=6)
    out, _ = O.orthogonalise(G, *coeffs, T)
    assert O.rel_frobenius(out, polar(G)) < 1e-12


def test_speedrun_coefficients_keep_singular_vectors():
    G = well_conditioned(32, 64, cond=5.0, seed=7)
    out, _ = O.orthogonalise(G, A, B, C, 5)
    assert O.rel_frobenius(polar(out), polar(G)) < 1e-12
    # ... but do not reach unit singular values
    assert O.rel_frobenius(out, polar(G)) > 0.05


# --- P6: the band the coefficients hold singular values in ------------------

def test_singular_value_band():
    # critical points of p solve p'(s) = a + 3 b s^2 + 5 c s^4 = 0 (a quadratic in s^2)
    r2 = np.roots([5 * C32, 3 * B32, A32])
    lo_pt, hi_pt = np.sqrt(np.sort(r2.real))
    assert abs(p_scalar(lo_pt) - 1.20237) < 1e-5 and abs(p_scalar(hi_pt) - 0.68183) < 1e-5
    band_lo, band_hi = p_scalar(hi_pt), p_scalar(lo_pt)
    # five steps bring every sigma0 in [1.52e-3, 1] into that band
    xs = np.linspace(1.52e-3, 1.0, 20001)
    ys = p_iter(xs, 5)
    assert ys.min() >= band_lo - 1e-12 and ys.max() <= band_hi + 1e-12
    # matrices whose normalised singular values are all >= 1.505e-3
    G = well_conditioned(48, 96, cond=100.0, seed=8)
    out, _ = O.orthogonalise(G, A, B, C, 5)
    sv = np.linalg.svd(out, compute_uv=False)
    assert sv.min() >= 0.68183 - 1e-6 and sv.max() <= 1.20237 + 1e-6


# --- P7: the polar factor maximises <G, O> over the spectral-norm unit ball --

def test_polar_attains_nuclear_norm():
    # overview page, "Reading guide": the orthogonalised update is steepest
    # descent under the spectral norm, so <G, polar(G)> = ||G||_* (sum of sigma).
    G = well_conditioned(20, 36, cond=4.0, seed=9) * 3.0
    out, _ = O.orthogonalise(G, 1.5, -0.5, 0.0, 20)
    nuclear = np.linalg.svd(G, compute_uv=False).sum()
    assert abs(np.sum(G * out) - nuclear) / nuclear < 1e-12


# --- P8: momentum recurrences on hand examples ------------------------------

def hand_gradients():
    g1 = np.arange(32, dtype=np.float64).reshape(4, 8) - 11.0
    g2 = (np.arange(32, dtype=np.float64).reshape(4, 8) % 5) * 3.0 - 4.0
    return g1, g2


def test_momentum_hand_example_mu_half():
    g1, g2 = hand_gradients()
    m0 = np.zeros((4, 8), np.float32)
    m1 = O.momentum_update(m0, g1, 0.5)
    m2 = O.momentum_update(m1, g2, 0.5)
    assert np.array_equal(m1, g1)
    assert np.array_equal(m2, 0.5 * g1 + g2)
    assert np.array_equal(O.nesterov_blend(g2, m2, 0.5, True), 0.25 * g1 + 1.5 * g2)
    assert np.array_equal(O.nesterov_blend(g2, m2, 0.5, False), 0.5 * g1 + g2)


def test_momentum_fp32_rounding_mu_095():
    g1, g2 = hand_gradients()
    mu32 = Fraction(float(np.float32(0.95)))
    assert float(mu32) == 0.949999988079071
    m1 = O.momentum_update(np.zeros((4, 8), np.float32), g1, 0.95)
    m2 = O.momentum_update(m1, g2, 0.95)
    assert np.array_equal(m1, g1.astype(np.float32))
    for i in range(4):
        for j in range(8):
            exact = mu32 * Fraction(float(g1[i, j])) + Fraction(float(g2[i, j]))
            # exact in fp64 (<= 34 significant bits), so one rounding to fp32
            assert m2[i, j] == np.float32(float(exact))
            assert m2.dtype == np.float32


def test_full_step_hand_example():
    # G = 3*[I4 | 0], zero momentum: M = G and U = (1+mu) G (Nesterov) or G, so
    # ||U|| = 6 (1+mu) or 6, every singular value of X0 is (||U||/2)/(||U|| + eps)
    # and O = p^5(sigma) [I4 | 0]; the weights move by -lr * s * O.
    e = np.hstack([np.eye(4), np.zeros((4, 4))])
    g = 3.0 * e
    w0 = np.full((4, 8), 0.25)
    for nesterov in (True, False):
        r = O.muon_step(w0, g, np.zeros((4, 8), np.float32), a=A, b=B, c=C, T=5, mu=0.95,
                        nesterov=nesterov, lr=0.1, scale=2.0)
        unorm = 6.0 * (1.0 + O.f32(0.95)) if nesterov else 6.0
        sigma = (unorm / 2.0) / (unorm + O.EPS)
        expect_o = p_iter(sigma, 5) * e
        assert abs(r.nu - unorm) < 1e-12
        assert O.rel_frobenius(r.O, expect_o) < 1e-13
        assert np.allclose(r.W, w0 - O.f32(0.1) * 2.0 * expect_o, rtol=0, atol=1e-15)
        assert np.array_equal(r.M, g.astype(np.float32))


def test_two_step_nesterov_versus_plain():
    g1, g2 = hand_gradients()
    kw = dict(a=A, b=B, c=C, T=5, mu=0.5, lr=1.0)
    z = np.zeros((4, 8))
    res_n = list(O.run_steps(z, [g1, g2], np.zeros((4, 8), np.float32), nesterov=True, **kw))
    res_p = list(O.run_steps(z, [g1, g2], np.zeros((4, 8), np.float32), nesterov=False, **kw))
    on, _ = O.orthogonalise(0.25 * g1 + 1.5 * g2, A, B, C, 5)
    op, _ = O.orthogonalise(0.5 * g1 + g2, A, B, C, 5)
    assert O.rel_frobenius(res_n[1].O, on) == 0.0
    assert O.rel_frobenius(res_p[1].O, op) == 0.0
    assert O.rel_frobenius(on, op) > 1e-3  # the flags are distinguishable at step 2
    # the weights accumulate -lr * O over the steps
    assert O.rel_frobenius(res_n[1].W, -(res_n[0].O + res_n[1].O)) < 1e-15


# --- P9: normalisation -------------------------------------------------------

def test_normalisation_trace():
    U = rng(10).standard_normal((33, 70)) * 0.02
    X0, nu = O.frobenius_normalise(U)
    assert abs(nu - np.linalg.norm(U)) < 1e-14
    assert abs(np.trace(X0 @ X0.T) - nu ** 2 / (nu + O.EPS) ** 2) < 1e-14


# --- P10: the pages' FLOP bound ---------------------------------------------

def test_flop_bound_from_pages():
    g = read_golden("flop_bound_record3.txt")
    T, m, Btok = g["T"], g["m"], g["B"]
    frac = O.ns_overhead_fraction([(m, m)], T, Btok)
    assert frac == Fraction(T * m, Btok)  # square m x m: exactly T m / B
    assert round(100 * frac, 1) == g["overhead_percent_approx"]
    # the whole GPT-2 small hidden set stays below the bound
    shapes = inputs.gpt2_hidden_shapes(12, 768)
    total = O.ns_overhead_fraction(shapes, T, Btok)
    assert total <= T * m / Btok
    assert abs(sum(O.ns_flops_dense(r, c, T) for r, c in shapes) - 1.6307e12) / 1.6307e12 < 1e-4
    # a tall n x m matrix costs T m (4n + 2m) / (6 n B) <= T m / B
    assert O.ns_overhead_fraction([(3072, 768)], T, Btok) == Fraction(T * 768 * (4 * 3072 + 2 * 768), 6 * 3072 * Btok)


def test_flop_counts_by_hand():
    # 2x3: m = 2, n = 3, T = 1.  Dense: XX^T 2*2*2*3=24, AA 2*8=16, BX 24 -> 64
    assert O.ns_flops_dense(2, 3, 1) == 64
    assert O.ns_flops_dense(3, 2, 1) == 64
    # distinct entries: XX^T 3 entries * 2*3 = 18; AA 3 entries * 2*2 = 12; BX 24 -> 54
    assert O.ns_flops_algorithmic(2, 3, 1) == 54


# --- P11: bf16 format of the inputs -----------------------------------------

def bf16_rne_bits(f32_bits: int) -> int:
    """Round an fp32 bit pattern to bf16 (8-bit exponent, 7-bit mantissa), ties to even."""
    exp = (f32_bits >> 23) & 0xFF
    if exp == 0xFF:  # inf / nan keep their top bits (nan stays nan)
        top = f32_bits >> 16
        return top | (0x40 if (f32_bits & 0x7FFFFF) else 0)
    low = f32_bits & 0xFFFF
    top = f32_bits >> 16
    if low > 0x8000 or (low == 0x8000 and (top & 1)):
        top += 1
    return top & 0xFFFF


def test_bf16_format_and_rounding():
    g = read_golden("bf16_format.txt")
    assert g["exponent_bits"] + g["mantissa_bits"] + 1 == 16
    assert torch.finfo(torch.bfloat16).eps == 2.0 ** -g["mantissa_bits"]
    r = rng(11)
    vals = np.concatenate([r.standard_normal(20000).astype(np.float32) * 0.02,
                           r.standard_normal(2000).astype(np.float32) * 1e30,
                           np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -1.0 - 2 ** -8,
                                     0.0, -0.0, 1e-40, 3.4e38], np.float32)])
    t = torch.from_numpy(vals).to(torch.bfloat16).view(torch.int16).numpy().astype(np.uint16)
    bits = vals.view(np.uint32)
    ref = np.array([bf16_rne_bits(int(b)) for b in bits], np.uint16)
    assert np.array_equal(t, ref)
    # the generators round through that same cast
    x = inputs.gaussian((64, 64), 0.02, 123, "cpu", torch.bfloat16)
    assert x.dtype == torch.bfloat16


# --- P12: per-iteration coefficient schedules (overview page, "Reading guide":
# later records tune the iteration's polynomials) -----------------------------

SCHEDULE = [(A, B, C), (A, B, C), (3.0, -3.2, 1.2), (15 / 8, -10 / 8, 3 / 8), (1.5, -0.5, 0.0)]


def schedule_via_svd(X0, schedule):
    """Closed form: every step maps the singular values through its own scalar polynomial."""
    U, S, Vt = np.linalg.svd(X0, full_matrices=False)
    for a, b, c in schedule:
        S = p_scalar(S, O.f32(a), O.f32(b), O.f32(c))
    return (U * S) @ Vt


@pytest.mark.parametrize("shape", [(40, 72), (72, 40), (9, 5)])
def test_schedule_matches_svd_closed_form(shape):
    G = rng(31).standard_normal(shape)
    X, transposed = O.to_short_side_first(G)
    X0, _ = O.frobenius_normalise(X)
    got = O.newton_schulz_schedule(X0, SCHEDULE)
    assert O.rel_frobenius(got, schedule_via_svd(X0, SCHEDULE)) < 1e-13
    Ofull, _ = O.orthogonalise(G, 0, 0, 0, 0, schedule=SCHEDULE)
    ref = schedule_via_svd(X0, SCHEDULE)
    assert O.rel_frobenius(Ofull, ref.T if transposed else ref) < 1e-13


def test_schedule_scalar_exact():
    """1x1 input: the composition of the steps' scalar maps, in exact rational arithmetic."""
    x = 0.375
    got = O.newton_schulz_schedule(np.array([[x]]), SCHEDULE)[0, 0]
    s = Fraction(x)
    for a, b, c in SCHEDULE:
        a, b, c = (Fraction(O.f32(v)) for v in (a, b, c))
        s = a * s + b * s ** 3 + c * s ** 5
    assert abs(got - float(s)) <= 1e-15 * max(1.0, abs(float(s)))


def test_schedule_aggressive_then_convergent_reaches_polar():
    """Three steps of the speedrun quintic put the singular values in its band; a
    convergent quintic tail then reaches the polar factor."""
    G = well_conditioned(48, 80, cond=5.0, seed=9)
    sched = [(A, B, C)] * 3 + [(15 / 8, -10 / 8, 3 / 8)] * 8
    out, _ = O.orthogonalise(G, 0, 0, 0, 0, schedule=sched)
    assert O.rel_frobenius(out, polar(G)) < 1e-10
    # the speedrun quintic alone does not get there
    out5, _ = O.orthogonalise(G, A, B, C, 5)
    assert O.rel_frobenius(out5, polar(G)) > 0.05


def test_schedule_of_one_triple_is_the_plain_iteration():
    G = rng(33).standard_normal((24, 40))
    X0, _ = O.frobenius_normalise(G)
    assert np.array_equal(O.newton_schulz_schedule(X0, [(A, B, C)] * 5), O.newton_schulz(X0, A, B, C, 5))
