"""fp64 CPU oracle of one Muon step -- TEST INFRASTRUCTURE, NOT PRODUCT CODE.

Only the tests, the package's smoke check and the benchmark's CPU-baseline leg
may import this module.  The product path (the HIP library and its Python
binding) never imports, calls or falls back to it.

What it computes, per hidden weight matrix and per step, in the order the
pages give the method:

1. momentum update of the gradient, Nesterov form
   ("NanoGPT Speedrun: The Ultimate Guide ...", section "Optimizer and
   Training Strategy Tuning": Muon orthogonalises the update after a Nesterov
   momentum step, and only for hidden-layer matrices);
2. replace that update by an approximation of its polar factor U V^T (the
   closest matrix with orthonormal rows or columns), computed with five
   Newton-Schulz steps
   ("The NanoGPT speedrun", paragraph "Six records account for most of the
   speedup", record #3);
3. scale the result and subtract it from the weights.

The pages name the iteration but not its polynomial, its normalisation or its
scalars.  The readings taken here (all passed in as arguments where they are
numbers) are:

* quintic step: A = X X^T, B = b A + c A^2, X <- a X + B X, with the short
  side first (X is transposed when the matrix has more rows than columns);
* X_0 = U / (||U||_F + eps), eps = 1e-7;
* momentum in SGD form, M <- mu M + G, Nesterov blend U = G + mu M, and the
  buffer stored at fp32 precision with one rounding per step (it is an fp32
  tensor on the device; an fp64 recurrence would drift from any honest fp32
  implementation);
* weight step W <- W - lr * s * O, s a per-matrix scale (default 1);
* every scalar is first rounded to fp32, since that is the value that crosses
  the library's C ABI.

Everything else is plain fp64: numpy matmul, no blocking, fusion or
reordering beyond the algebra above.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional, Tuple

import numpy as np

EPS = 1e-7


def f32(x: float) -> float:
    """The fp32 value a float argument takes when it crosses the C ABI."""
    return float(np.float32(x))


def as_f64(t) -> np.ndarray:
    """Exact fp64 copy of a numpy array or CPU torch tensor (bf16/fp32)."""
    if hasattr(t, "detach"):  # torch tensor: widen through fp32, which is exact for bf16
        import torch  # local import: the oracle itself is numpy-only

        return t.detach().to("cpu", torch.float64).numpy()
    return np.asarray(t, dtype=np.float64)


def momentum_update(M: np.ndarray, G: np.ndarray, mu: float) -> np.ndarray:
    """M <- fl32(mu*M + G): the momentum buffer after this step's gradient.

    Guide page, "Optimizer and Training Strategy Tuning" (momentum precedes
    orthogonalisation).  The product and the sum are formed in fp64 (the
    product of two fp32 numbers is exact there) and the result is rounded
    once to fp32, the buffer's storage precision.
    """
    mu32 = f32(mu)
    return (mu32 * np.asarray(M, np.float64) + np.asarray(G, np.float64)).astype(np.float32)


def nesterov_blend(G: np.ndarray, M_new: np.ndarray, mu: float, nesterov: bool) -> np.ndarray:
    """The update that gets orthogonalised: G + mu*M (Nesterov) or M (plain momentum)."""
    if nesterov:
        return np.asarray(G, np.float64) + f32(mu) * np.asarray(M_new, np.float64)
    return np.asarray(M_new, np.float64).copy()


def to_short_side_first(U: np.ndarray) -> Tuple[np.ndarray, bool]:
    """Return (X, transposed): X has no more rows than columns."""
    if U.shape[0] > U.shape[1]:
        return U.T.copy(), True
    return U.copy(), False


def frobenius_normalise(X: np.ndarray, eps: float = EPS) -> Tuple[np.ndarray, float]:
    """X / (||X||_F + eps), and ||X||_F."""
    nu = float(np.sqrt(np.sum(X * X)))
    return X / (nu + eps), nu


def newton_schulz(X0: np.ndarray, a: float, b: float, c: float, T: int) -> np.ndarray:
    """T quintic Newton-Schulz steps on a short-side-first X_0 (rows <= cols).

    Speedrun overview page, "Six records ..." (record #3): the normalised update
    is driven towards its polar factor U V^T by Newton-Schulz
    steps.  Each step: A = X X^T, B = b A + c A A, X <- a X + B X.
    """
    a, b, c = f32(a), f32(b), f32(c)
    X = np.asarray(X0, np.float64)
    for _ in range(T):
        A = X @ X.T
        B = b * A + c * (A @ A)
        X = a * X + B @ X
    return X


def newton_schulz_schedule(X0: np.ndarray, schedule) -> np.ndarray:
    """Newton-Schulz steps with their own polynomial each: step t uses schedule[t] = (a, b, c).

    Speedrun overview page, paragraph "Reading guide": later records tune the
    iteration's polynomials (Polar Express).  The pages give no values, so the
    schedule is an argument; every step is the quintic step above with its own
    (a, b, c).
    """
    X = np.asarray(X0, np.float64)
    for a, b, c in schedule:
        a, b, c = f32(a), f32(b), f32(c)
        A = X @ X.T
        B = b * A + c * (A @ A)
        X = a * X + B @ X
    return X


def orthogonalise(U: np.ndarray, a: float, b: float, c: float, T: int,
                  eps: float = EPS, schedule=None) -> Tuple[np.ndarray, float]:
    """Short side first, normalise, iterate, and return O in U's orientation (and ||U||_F).

    ``schedule`` (a list of (a, b, c)) replaces a, b, c and T when given.
    """
    X, transposed = to_short_side_first(np.asarray(U, np.float64))
    X0, nu = frobenius_normalise(X, eps)
    X = newton_schulz(X0, a, b, c, T) if schedule is None else newton_schulz_schedule(X0, schedule)
    return (X.T.copy() if transposed else X), nu


@dataclass
class StepResult:
    W: np.ndarray        # weights after the step (fp64)
    M: np.ndarray        # momentum buffer after the step (fp32 values)
    O: np.ndarray        # orthogonalised update, gradient orientation (fp64)
    nu: float            # ||U||_F


def muon_step(W: np.ndarray, G: np.ndarray, M: np.ndarray, *, a: float = 0.0, b: float = 0.0, c: float = 0.0,
              T: int = 0, mu: float, nesterov: bool, lr: float, scale: float = 1.0,
              eps: float = EPS, schedule=None) -> StepResult:
    """One Muon step on one hidden matrix: momentum, orthogonalise, apply.

    W, G, M are the exact values the device sees (fp32 / bf16 / fp32).
    The weight step is W - lr*s*O in fp64; s <= 0 selects the default s = 1.
    ``schedule`` (one (a, b, c) per iteration) replaces a, b, c and T when given.
    """
    G64 = as_f64(G)
    M_new = momentum_update(as_f64(M), G64, mu)
    U = nesterov_blend(G64, M_new, mu, nesterov)
    O, nu = orthogonalise(U, a, b, c, T, eps, schedule=schedule)
    s = 1.0 if scale <= 0 else f32(scale)
    W_new = as_f64(W) - f32(lr) * s * O
    return StepResult(W_new, M_new, O, nu)


def run_steps(W0, grads_per_step, M0, **kw):
    """Apply ``muon_step`` over a sequence of gradients; yields StepResult per step."""
    W = as_f64(W0)
    M = np.asarray(as_f64(M0), np.float32)
    for G in grads_per_step:
        r = muon_step(W, G, M, **kw)
        W, M = r.W, r.M
        yield r


# --- work model -------------------------------------------------------------

def ns_flops_dense(rows: int, cols: int, T: int) -> int:
    """FLOPs of T Newton-Schulz steps counted as dense products.

    With short side m and long side n: X X^T is 2 m^2 n, A A is 2 m^3 and
    B X is 2 m^2 n.  This is the model behind the speedrun overview page's
    bound of T m / B extra FLOPs (paragraph "Six records ...", record #3).
    """
    m, n = min(rows, cols), max(rows, cols)
    return T * (4 * m * m * n + 2 * m ** 3)


def ns_flops_algorithmic(rows: int, cols: int, T: int) -> int:
    """FLOPs of T steps counting only the distinct entries of the symmetric products.

    X X^T and A A are symmetric: m(m+1)/2 distinct entries, each a length-n
    (resp. length-m) dot product of 2n (2m) FLOPs.  B X is a full product.
    """
    m, n = min(rows, cols), max(rows, cols)
    return T * (m * (m + 1) * n + m * m * (m + 1) + 2 * m * m * n)


def training_flops(params: int, tokens: int) -> int:
    """The usual 6 * params * tokens count of one forward+backward over a batch."""
    return 6 * params * tokens


def ns_overhead_fraction(shapes, T: int, tokens_per_step: int) -> float:
    """Dense Newton-Schulz FLOPs of a set of matrices over their training FLOPs."""
    ns = sum(ns_flops_dense(r, c, T) for r, c in shapes)
    tr = training_flops(sum(r * c for r, c in shapes), tokens_per_step)
    return ns / tr


def rel_frobenius(x: np.ndarray, ref: np.ndarray) -> float:
    """||x - ref||_F / ||ref||_F (0 when both are 0)."""
    x = np.asarray(x, np.float64)
    ref = np.asarray(ref, np.float64)
    den = float(np.linalg.norm(ref))
    num = float(np.linalg.norm(x - ref))
    if den == 0.0:
        return 0.0 if num == 0.0 else float("inf")
    return num / den
