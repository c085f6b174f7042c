"""Plain fp64 CPU oracle for batched Newton–Schulz (NS) orthogonalization.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports, calls or runs
this module; only the tests, the package smoke check and the bench's CPU
baseline do.  It shares no code with the HIP library.

What it computes, step by step, in the order and notation of the pages
("Dion3: Full-stack orthogonal updates", Sections 2.2, 4 and Appendix B.2.3;
the "muon" kernel card, "How it works"):

  * ``normalize``      X <- X / (s (||X||_F + eps))              (Alg. 1 / Alg. 3 step 2)
  * ``standard_ns``    X <- a X + (b A + c A^2) X with A = X X^T   (Alg. 1)
  * ``gram_ns``        R = X X^T, Q = I, loop with restarts       (Alg. 3, App. B.2)
  * ``orthogonalize``  the bucket wrapper: transpose so the short side leads,
                       pick the mode (square -> standard), normalize, iterate,
                       transpose back.

Every matrix product is ``numpy.matmul`` in float64; nothing is blocked, fused
or reordered beyond what the algorithms state, so each line can be checked
against the pages by eye.

Readings of points the pages leave open:
  * safety factor s: applied once, at normalization (X / (s (||X||_F + eps))).
    The per-polynomial form p(x/s) of Appendix B.2.2 equals this scaling
    applied at every step; it is obtained by passing rescaled coefficients.
  * restart_after = r: the restart happens at the top of iteration r + 1
    (Alg. 3 restarts at the top of step 3, i.e. r = 2).  r = 0, or r >= T, means no
    restart (Alg. 2 with the implicit a*I form of Appendix B.2.3).
  * square matrices (m == n) in "gram" mode run standard NS (Section 4.1, last
    paragraph).
  * a rank-deficient input keeps its zero singular values at zero (odd
    polynomials); no pseudo-inverse is needed.

Pins (tests/test_oracle_pins.py) tie this module to facts outside itself:
brute-force SVD of tiny matrices against the composed scalar polynomial,
unchanged singular vectors, Gram == standard in fp64, every restart location
agreeing, closed forms for diagonal and orthonormal-row inputs, transpose /
orthogonal / scale invariances, and the FLOP percentages the pages print.
"""
from __future__ import annotations

from typing import Sequence

import numpy as np

EPS = 1e-7  # Alg. 1 / Alg. 3 step 2


def _coeff_list(coeffs, steps: int):
    """Per-step (a_t, b_t, c_t): one triple reused, or `steps` triples."""
    c = np.asarray(coeffs, dtype=np.float64).reshape(-1, 3)
    if c.shape[0] == 1:
        c = np.repeat(c, steps, axis=0)
    if c.shape[0] != steps:
        raise ValueError("coeffs must hold 3 or 3*steps values")
    return [tuple(row) for row in c]


def normalize(X: np.ndarray, safety: float = 1.0, eps: float = EPS) -> np.ndarray:
    """X / (s (||X||_F + eps)): singular values into [0, 1/s].

    Dion3 paper, Alg. 1 and Alg. 3, step 2 (eps = 1e-7); safety factor s of
    Appendix B.2.2 ("Safety Factors") applied once, here.
    """
    nu = np.sqrt(np.sum(X * X))
    return X / (safety * (nu + eps))


def gram(X: np.ndarray) -> np.ndarray:
    """The Gram matrix X X^T of the short side (n x n)."""
    return X @ X.T


def quadratic(A: np.ndarray, b: float, c: float) -> np.ndarray:
    """b A + c A^2: the matrix polynomial h_t(A) = a + b A + c A^2 without its
    a*I term, which every caller applies on its own (Dion3 paper, App. B.2.3)."""
    return b * A + c * (A @ A)


def standard_ns(X: np.ndarray, coeffs, steps: int = 5) -> np.ndarray:
    """Standard quintic Newton–Schulz on an already normalized X (n <= m).

    Dion3 paper, Section 2.2, Algorithm 1: every step applies the odd
    quintic p_t(X) = a_t X + b_t (X X^T) X + c_t (X X^T)^2 X, i.e.
    X <- a_t X + h(X X^T) X with h the quadratic part above.
    """
    for a, b, c in _coeff_list(coeffs, steps):
        X = a * X + quadratic(gram(X), b, c) @ X
    return X


def _restart_steps(steps: int, restart_after: int, restarts):
    """Steps t at whose top the iteration restarts.  ``restarts`` (any
    iterable of steps 2..T) overrides the single ``restart_after``."""
    if restarts is not None:
        rs = sorted(set(int(t) for t in restarts))
        if any(t < 2 or t > steps for t in rs):
            raise ValueError("restart steps must lie in 2..steps")
        return rs
    return [restart_after + 1] if 1 <= restart_after < steps else []


def gram_ns(X: np.ndarray, coeffs, steps: int = 5, restart_after: int = 2,
            gram_shift: float = 0.0, restarts=None) -> np.ndarray:
    """Gram Newton–Schulz with restarts, on an already normalized X (n <= m).

    Dion3 paper, Section 4.2, Algorithm 3 (stabilized Gram NS), with the a*I
    terms kept out of Z as in Appendix B.2.3:
        R_0 <- X X^T ;  Q_0 <- I
        for t = 1..T:
            if t == restart_after + 1:  X <- Q X ;  R <- X X^T ;  Q <- I
            Z_t    <- b_t R + c_t R^2
            Q_t    <- Q Z_t + a_t Q
            (RZ)_t <- R Z_t + a_t R
            R_t    <- Z_t (RZ)_t + a_t (RZ)_t
        return Q_T X
    restart_after = 0 (or >= T) gives Algorithm 2 without a restart.
    ``restarts`` lists several restart steps: Appendix B.2 repeats the
    restart to reach any X_T, and B.2.1 sweeps schedules with more than one.

    ``gram_shift`` subtracts shift*I each time a Gram matrix is formed, the
    simulated spurious eigenvalue of Appendix B.2.1 (there: 4e-4); 0 normally.
    """
    I = np.eye(X.shape[0])
    R = gram(X) - gram_shift * I
    Q = I.copy()
    at = _restart_steps(steps, restart_after, restarts)
    for t, (a, b, c) in enumerate(_coeff_list(coeffs, steps), start=1):
        if t in at:
            X = Q @ X
            R = gram(X) - gram_shift * I
            Q = I.copy()
        Z = quadratic(R, b, c)
        Q = Q @ Z + a * Q
        RZ = R @ Z + a * R
        R = Z @ RZ + a * RZ
    return Q @ X


def naive_gram_ns(X: np.ndarray, coeffs, steps: int = 5,
                  r0_shift: float = 0.0) -> np.ndarray:
    """Algorithm 2 as printed (explicit a*I inside Z), optional spurious shift.

    Dion3 paper, Section 4, Algorithm 2: R_0 = X X^T and Q_0 = I, then each
    step forms Z_t = h_t(R) = a I + b R + c R^2 and updates Q by Q Z_t and R by
    Z_t R Z_t; the output is Q_T X.
    ``r0_shift`` subtracts shift*I from R_0, the simulated spurious negative
    eigenvalue of Appendix B.2.1 (about -4e-4).
    """
    I = np.eye(X.shape[0])
    R = gram(X) - r0_shift * I
    Q = I.copy()
    for a, b, c in _coeff_list(coeffs, steps):
        Z = a * I + quadratic(R, b, c)   # h_t(R) with its a*I term inside Z
        Q, R = Q @ Z, Z @ R @ Z
    return Q @ X


def ns_matrix(Y: np.ndarray, steps: int, coeffs, mode: str = "gram",
              restart_after: int = 2, safety: float = 1.0, eps: float = EPS,
              restarts=None) -> np.ndarray:
    """One R x C matrix: transpose so n <= m, normalize, iterate, transpose back.

    Transposition: Alg. 1 takes X in R^{n x m} with n <= m; the "muon" kernel
    card transposes a tall matrix so that the products contract over its
    long side.
    Mode: square matrices always run standard NS (Dion3 paper, Section 4.1).
    """
    Y = np.asarray(Y, dtype=np.float64)
    tr = Y.shape[0] > Y.shape[1]
    X = Y.T if tr else Y
    n, m = X.shape
    X = normalize(X, safety, eps)
    if mode == "standard" or n == m:
        X = standard_ns(X, coeffs, steps)
    elif mode == "gram":
        X = gram_ns(X, coeffs, steps, restart_after, restarts=restarts)
    else:
        raise ValueError(f"unknown mode {mode!r}")
    return X.T if tr else X


def orthogonalize(Gs: np.ndarray, steps: int = 5, coeffs=(3.4445, -4.7750, 2.0315),
                  mode: str = "gram", restart_after: int = 2, safety: float = 1.0,
                  eps: float = EPS, restarts=None) -> np.ndarray:
    """Bucket [G, R, C] -> [G, R, C], each matrix on its own (fp64 throughout).

    The "muon" kernel card ("How it works") stacks a shape bucket into one
    [G, R, C] tensor; every matrix is orthogonalized independently.
    """
    Gs = np.asarray(Gs, dtype=np.float64)
    out = np.empty_like(Gs)
    for g in range(Gs.shape[0]):
        out[g] = ns_matrix(Gs[g], steps, coeffs, mode, restart_after, safety, eps, restarts)
    return out


# ---------------------------------------------------------------------------
# Scalar views (Dion3 paper, Section 2.2 and Theorem 2)
# ---------------------------------------------------------------------------

def composed_polynomial(x, coeffs, steps: int = 5) -> np.ndarray:
    """(p_T o ... o p_1)(x) with p_t(x) = a_t x + b_t x^3 + c_t x^5 (Section 2.2)."""
    x = np.asarray(x, dtype=np.float64)
    for a, b, c in _coeff_list(coeffs, steps):
        x = a * x + b * x ** 3 + c * x ** 5
    return x


def theorem2_q(x, coeffs, steps: int = 5) -> np.ndarray:
    """q_T of Theorem 2: r_0 = x^2, q_0 = 1, z_t = h_t(r_{t-1}),
    r_t = r_{t-1} z_t^2, q_t = q_{t-1} z_t, with h_t(y) = a_t + b_t y + c_t y^2."""
    x = np.asarray(x, dtype=np.float64)
    r = x * x
    q = np.ones_like(x)
    for a, b, c in _coeff_list(coeffs, steps):
        z = a + b * r + c * r * r
        r = r * z * z
        q = q * z
    return q


# ---------------------------------------------------------------------------
# FLOP models printed on the pages (n = short side, alpha = m / n)
# ---------------------------------------------------------------------------

def flops_standard(n: int, m: int, T: int = 5) -> float:
    """2T(2 alpha + 1) n^3 = T (4 m n^2 + 2 n^3): Dion3 paper, Section 2.2."""
    return float(T) * (4.0 * m * n * n + 2.0 * n ** 3)


def flops_standard_symmetric(n: int, m: int, T: int = 5) -> float:
    """T (3 alpha + 1) n^3: Dion3 paper, Section 2.3 (symmetric GEMMs)."""
    return float(T) * (3.0 * m * n * n + n ** 3)


def flops_gram_naive(n: int, m: int, T: int = 5) -> float:
    """(4T + 3 alpha - 3) n^3: Dion3 paper, Section 4.1."""
    return 4.0 * T * n ** 3 + 3.0 * m * n * n - 3.0 * n ** 3


def flops_gram_stable(n: int, m: int, T: int = 5, restarts: int = 1) -> float:
    """(4T + 6 alpha - 6) n^3 for one restart: Section 4.1 plus 3(alpha-1)n^3 per
    restart (Section 4.2); written out on the "Gram Newton–Schulz" blog post."""
    return flops_gram_naive(n, m, T) + restarts * 3.0 * (m * n * n - n ** 3)
