"""Pins of the fp64 oracle to facts outside itself (CPU only).

Each test checks the oracle against something the pages or the mathematics fix
independently of the oracle's own code: LAPACK SVDs of tiny matrices, the
scalar recurrences of Theorem 2, closed forms, invariances, and the FLOP
figures printed on the pages (tests/golden/flop_savings.json).
"""
import json
import os

import numpy as np
import pytest

import oracle
from synth import COEFFS_CLASSIC, COEFFS_MUON, conditioning_matrix, make

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rel(a, b):
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def svd_expected(Y, steps, coeffs, safety, eps=oracle.EPS):
    """U diag(p_T o..o p_1(sigma / (s (nu + eps)))) V^T from LAPACK's SVD of Y.

    The Frobenius norm nu is taken from the singular values (sqrt of the sum
    of their squares), not from the entries, so nothing is shared with the
    oracle's normalize step.  Dion3 paper, Section 2.2 (spectral view).
    """
    U, S, Vt = np.linalg.svd(Y, full_matrices=False)
    nu = np.sqrt(np.sum(S ** 2))
    x = S / (safety * (nu + eps))
    # composed polynomial written out here independently of the oracle
    c = np.asarray(coeffs, dtype=np.float64).reshape(-1, 3)
    if c.shape[0] == 1:
        c = np.repeat(c, steps, axis=0)
    for a, b, cc in c:
        x = a * x + b * x ** 3 + cc * x ** 5
    return (U * x[None, :]) @ Vt


TINY = [(2, 3), (4, 8), (8, 32), (16, 16), (24, 8), (5, 13), (1, 7)]


# --------------------------------------------------------------------------
# Theorem 2 and the scalar polynomial
# --------------------------------------------------------------------------

@pytest.mark.parametrize("coeffs", [COEFFS_MUON, COEFFS_CLASSIC])
def test_theorem2_scalar_identity(coeffs):
    """(p_T o..o p_1)(x) = q_T x on 10^4 points of [0, 1] (Theorem 2)."""
    x = np.linspace(0.0, 1.0, 10_001)
    lhs = oracle.composed_polynomial(x, coeffs, 5)
    rhs = oracle.theorem2_q(x, coeffs, 5) * x
    assert np.max(np.abs(lhs - rhs)) <= 5e-14  # a few ulps of values up to ~1.2


def test_classic_polynomial_fixed_point_and_convergence():
    """(15/8, -10/8, 3/8): p(1) = 1 exactly, and iterating drives (0, 1] to 1.

    Appendix B.1.1 uses these coefficients; p(1) = 15/8 - 10/8 + 3/8 = 1 and
    p'(1) = 0, so it is the classic quintic Newton-Schulz map (textbook).
    """
    assert oracle.composed_polynomial(1.0, COEFFS_CLASSIC, 1) == 1.0
    x = np.array([0.02, 0.1, 0.5, 0.9, 1.0])
    y = oracle.composed_polynomial(x, COEFFS_CLASSIC, 40)
    assert np.max(np.abs(y - 1.0)) <= 1e-12
    # q_t -> 1/x (corollary of Theorem 2)
    q = oracle.theorem2_q(x, COEFFS_CLASSIC, 40)
    assert np.max(np.abs(q * x - 1.0)) <= 1e-12


def test_muon_coefficients_loose_by_design():
    """The fixed Muon triple pulls singular values toward one only loosely
    ("muon" kernel card): one step maps 1 to a + b + c = 0.701, and after 5
    steps the image of [0.01, 1] is a band around one, about [0.68, 1.14]."""
    assert abs(oracle.composed_polynomial(1.0, COEFFS_MUON, 1) - 0.701) <= 1e-12
    x = np.linspace(1e-2, 1.0, 2001)
    y = oracle.composed_polynomial(x, COEFFS_MUON, 5)
    assert y.min() > 0.65 and y.max() < 1.2
    assert np.max(np.abs(y - 1.0)) > 0.1


# --------------------------------------------------------------------------
# Spectral map: brute-force SVD on tiny matrices
# --------------------------------------------------------------------------

@pytest.mark.parametrize("shape", TINY)
@pytest.mark.parametrize("mode", ["standard", "gram"])
@pytest.mark.parametrize("safety", [1.0, 1.05])
def test_spectral_map_tiny(shape, mode, safety):
    """Output = U p(Sigma/(s(nu+eps))) V^T: singular vectors kept, values mapped
    by the composed polynomial (Dion3 paper, Section 2.2)."""
    rng = np.random.default_rng(hash((shape, mode)) % 2**32)
    Y = rng.standard_normal(shape)
    out = oracle.ns_matrix(Y, 5, COEFFS_MUON, mode, 2, safety)
    exp = svd_expected(Y, 5, COEFFS_MUON, safety)
    assert rel(out, exp) <= 1e-12


@pytest.mark.parametrize("mode", ["standard", "gram"])
def test_singular_vectors_unchanged(mode):
    """||offdiag(U^T Y V)||_F / ||Y||_F <= 1e-12 (Section 2.2)."""
    rng = np.random.default_rng(7)
    X = rng.standard_normal((16, 40))
    U, S, Vt = np.linalg.svd(X, full_matrices=False)
    Y = oracle.ns_matrix(X, 5, COEFFS_MUON, mode, 2, 1.0)
    D = U.T @ Y @ Vt.T
    off = D - np.diag(np.diag(D))
    assert np.linalg.norm(off) / np.linalg.norm(Y) <= 1e-12


@pytest.mark.parametrize("mode", ["standard", "gram"])
def test_rank_deficient_keeps_zero_singular_values(mode):
    """A rank-3 8x32 input gives a rank-3 output whose null space is the input's
    (odd polynomials keep 0 at 0; the blog post's compact-SVD remark)."""
    rng = np.random.default_rng(3)
    X = rng.standard_normal((8, 3)) @ rng.standard_normal((3, 32))
    Y = oracle.ns_matrix(X, 5, COEFFS_MUON, mode, 2, 1.0)
    s = np.linalg.svd(Y, compute_uv=False)
    assert s[3:].max() <= 1e-12 * s[0]
    # Y annihilates the orthogonal complement of X's row space
    _, _, Vt = np.linalg.svd(X)
    null = Vt[3:].T
    assert np.linalg.norm(Y @ null) <= 1e-12 * np.linalg.norm(Y)
    assert rel(Y, svd_expected(X, 5, COEFFS_MUON, 1.0)) <= 1e-10


# --------------------------------------------------------------------------
# Gram NS == standard NS in fp64, every restart location
# --------------------------------------------------------------------------

def test_gram_equals_standard_single_128x512():
    """fp64 Gram NS equals fp64 standard NS to <= 1e-12 relative (Section 4:
    'mathematically identical'), on the seed-0 128x512 matrix."""
    Y = make("single_1x128x512_f32")[0].double().numpy()
    a = oracle.ns_matrix(Y, 5, COEFFS_MUON, "standard", 2, 1.0)
    b = oracle.ns_matrix(Y, 5, COEFFS_MUON, "gram", 2, 1.0)
    assert rel(b, a) <= 1e-12


@pytest.mark.parametrize("restart_after", [0, 1, 2, 3, 4, 5, 9])
def test_every_restart_location_is_exact(restart_after):
    """A restart changes nothing in exact arithmetic (Section 4.2): every
    location, and none, agrees with standard NS in fp64."""
    rng = np.random.default_rng(restart_after)
    X = oracle.normalize(rng.standard_normal((24, 96)), 1.05)
    a = oracle.standard_ns(X, COEFFS_MUON, 5)
    b = oracle.gram_ns(X, COEFFS_MUON, 5, restart_after)
    assert rel(b, a) <= 1e-12


@pytest.mark.parametrize("cls", ["gaussian", "ill_conditioned", "low_rank", "heavy_tailed",
                                 "scaled_up", "scaled_down", "near_orthogonal"])
def test_gram_equals_standard_conditionings(cls):
    """The seven conditioning classes of the 'muon' kernel card, 96x384."""
    rng = np.random.default_rng(2)
    Y = conditioning_matrix(cls, rng, 96, 384)
    a = oracle.ns_matrix(Y, 5, COEFFS_MUON, "standard", 2, 1.05)
    b = oracle.ns_matrix(Y, 5, COEFFS_MUON, "gram", 2, 1.05)
    assert rel(b, a) <= 1e-12


def test_per_step_coefficients():
    """Distinct (a_t, b_t, c_t) per step: Gram and standard still agree and
    match the SVD spectral map (Alg. 1 takes {(a_t, b_t, c_t)}_{t=1..T})."""
    coeffs = [3.4445, -4.7750, 2.0315, 15 / 8, -10 / 8, 3 / 8, 2.0, -1.5, 0.5]
    rng = np.random.default_rng(9)
    Y = rng.standard_normal((12, 30))
    a = oracle.ns_matrix(Y, 3, coeffs, "standard", 1, 1.0)
    b = oracle.ns_matrix(Y, 3, coeffs, "gram", 1, 1.0)
    assert rel(b, a) <= 1e-12
    assert rel(a, svd_expected(Y, 3, coeffs, 1.0)) <= 1e-12


# --------------------------------------------------------------------------
# Closed forms
# --------------------------------------------------------------------------

@pytest.mark.parametrize("mode", ["standard", "gram"])
def test_diagonal_block_closed_form(mode):
    """X = [diag(d) | 0] -> [diag(p(d/(s(nu+eps)))) | 0] exactly in form."""
    d = np.array([3.0, 1.0, 0.5, 0.25, 2.0])
    X = np.zeros((5, 12))
    X[:, :5] = np.diag(d)
    s = 1.05
    x = d / (s * (np.sqrt(np.sum(d ** 2)) + oracle.EPS))
    p = x.copy()
    for _ in range(5):
        a, b, c = COEFFS_MUON
        p = a * p + b * p ** 3 + c * p ** 5
    exp = np.zeros_like(X)
    exp[:, :5] = np.diag(p)
    Y = oracle.ns_matrix(X, 5, COEFFS_MUON, mode, 2, s)
    assert np.max(np.abs(Y - exp)) <= 1e-14


def test_unit_row_vector_is_fixed_by_classic_coefficients():
    """n = 1: x/||x|| has singular value 1, a fixed point of the classic
    quintic (p(1) = 1, p'(1) = 0), so the output is x/||x|| (App. B.1.1)."""
    rng = np.random.default_rng(4)
    x = rng.standard_normal((1, 50)) * 3.0
    Y = oracle.ns_matrix(x, 5, COEFFS_CLASSIC, "gram", 2, 1.0)
    assert np.max(np.abs(Y - x / np.linalg.norm(x))) <= 1e-13


@pytest.mark.parametrize("mode", ["standard", "gram"])
def test_orthonormal_rows_closed_form(mode):
    """c * (orthonormal rows): X0 = X/(s (nu + eps)) has every singular value
    sigma = c / (s (c sqrt(n) + eps)), so the output is p(sigma)/sigma * X0."""
    rng = np.random.default_rng(5)
    n, m, c, s = 6, 20, 2.5, 1.05
    q, _ = np.linalg.qr(rng.standard_normal((m, n)))
    X = c * q.T
    sigma = c / (s * (c * np.sqrt(n) + oracle.EPS))
    p = sigma
    for _ in range(5):
        a, b, cc = COEFFS_MUON
        p = a * p + b * p ** 3 + cc * p ** 5
    exp = (p / c) * X
    Y = oracle.ns_matrix(X, 5, COEFFS_MUON, mode, 2, s)
    assert rel(Y, exp) <= 1e-13


def test_zero_matrix_gives_zero():
    Y = oracle.ns_matrix(np.zeros((4, 9)), 5, COEFFS_MUON, "gram", 2, 1.05)
    assert np.all(Y == 0.0)


# --------------------------------------------------------------------------
# Invariances
# --------------------------------------------------------------------------

@pytest.mark.parametrize("mode", ["standard", "gram"])
def test_transpose_invariance(mode):
    """NS(X^T) = NS(X)^T: the bucket wrapper transposes tall matrices so the
    short side leads ('muon' kernel card; Alg. 1 takes n <= m)."""
    rng = np.random.default_rng(6)
    Y = rng.standard_normal((40, 11))
    a = oracle.ns_matrix(Y, 5, COEFFS_MUON, mode, 2, 1.05)
    b = oracle.ns_matrix(Y.T, 5, COEFFS_MUON, mode, 2, 1.05)
    assert np.array_equal(a, b.T)
    assert rel(a, svd_expected(Y, 5, COEFFS_MUON, 1.05)) <= 1e-12


@pytest.mark.parametrize("mode", ["standard", "gram"])
def test_orthogonal_equivariance(mode):
    """NS(U X V) = U NS(X) V for orthogonal U, V (polar is equivariant)."""
    rng = np.random.default_rng(8)
    X = rng.standard_normal((10, 26))
    U, _ = np.linalg.qr(rng.standard_normal((10, 10)))
    V, _ = np.linalg.qr(rng.standard_normal((26, 26)))
    a = oracle.ns_matrix(U @ X @ V, 5, COEFFS_MUON, mode, 2, 1.0)
    b = U @ oracle.ns_matrix(X, 5, COEFFS_MUON, mode, 2, 1.0) @ V
    assert rel(a, b) <= 1e-12


def test_scale_invariance_up_to_eps():
    """NS(c X) = NS(X) up to the eps in the normalization (~1e-7 relative)."""
    rng = np.random.default_rng(10)
    X = rng.standard_normal((12, 48))
    a = oracle.ns_matrix(X, 5, COEFFS_MUON, "gram", 2, 1.05)
    b = oracle.ns_matrix(4.0 * X, 5, COEFFS_MUON, "gram", 2, 1.05)
    assert rel(a, b) <= 1e-6


def test_grouped_equals_single_bitwise():
    """Batching a shape bucket does not change any matrix ('muon' kernel card,
    Correctness: grouped and per-matrix agree)."""
    Gs = make("gpt2s_mlp_42x768x3072_f16", G=7, R=24, C=80).double().numpy()
    out = oracle.orthogonalize(Gs, 5, COEFFS_MUON, "gram", 2, 1.05)
    for g in range(Gs.shape[0]):
        one = oracle.orthogonalize(Gs[g:g + 1], 5, COEFFS_MUON, "gram", 2, 1.05)
        assert np.array_equal(out[g], one[0])


# --------------------------------------------------------------------------
# Restart location and the simulated spurious eigenvalue (Appendix B.2.1)
# --------------------------------------------------------------------------

@pytest.mark.parametrize("restart_after", [0, 1, 2, 3])
def test_shifted_gram_matches_scalar_model(restart_after):
    """With -delta*I injected at every Gram formation, each eigen-direction
    still evolves on its own (the shift shares U), so the output is
    U diag(f(sigma)) V^T with f from the scalar recurrences of Theorem 2:
    r = sigma^2 - delta, q = 1; at the restart x <- q x, r <- x^2 - delta,
    q <- 1; output q x.  This pins where the restart happens."""
    delta = 4e-4
    rng = np.random.default_rng(12)
    X = oracle.normalize(rng.standard_normal((8, 24)) @ np.diag(np.logspace(0, -2, 24)), 1.0)
    U, S, Vt = np.linalg.svd(X, full_matrices=False)
    x = S.copy()
    r = x * x - delta
    q = np.ones_like(x)
    for t in range(1, 6):
        if restart_after >= 1 and t == restart_after + 1:
            x = q * x
            r = x * x - delta
            q = np.ones_like(x)
        a, b, c = COEFFS_MUON
        z = a + b * r + c * r * r
        r = r * z * z
        q = q * z
    exp = (U * (q * x)[None, :]) @ Vt
    got = oracle.gram_ns(X, COEFFS_MUON, 5, restart_after, gram_shift=delta)
    assert rel(got, exp) <= 1e-11


@pytest.mark.parametrize("restarts", [[2], [3, 5], [2, 4, 6, 8], [5, 10], list(range(2, 11))])
def test_several_restarts_are_exact(restarts):
    """Repeating the restart (Appendix B.2: restart every few iterations to
    reach any X_T) still changes nothing in exact arithmetic: T = 10 steps with
    the restarts listed agree with standard NS in fp64.  Restarting at every
    step is standard NS written through Q = Z + aI."""
    rng = np.random.default_rng(31)
    X = oracle.normalize(rng.standard_normal((20, 70)), 1.05)
    coeffs = [3.4445, -4.7750, 2.0315] * 5 + [15 / 8, -10 / 8, 3 / 8] * 5
    a = oracle.standard_ns(X, coeffs, 10)
    b = oracle.gram_ns(X, coeffs, 10, restarts=restarts)
    assert rel(b, a) <= 1e-11


def test_restart_list_matches_restart_after():
    rng = np.random.default_rng(32)
    X = oracle.normalize(rng.standard_normal((12, 40)), 1.0)
    for r in (1, 2, 3, 4):
        assert np.array_equal(oracle.gram_ns(X, COEFFS_MUON, 5, r), oracle.gram_ns(X, COEFFS_MUON, 5, 0, restarts=[r + 1]))
    with pytest.raises(ValueError):
        oracle.gram_ns(X, COEFFS_MUON, 5, restarts=[1])
    with pytest.raises(ValueError):
        oracle.gram_ns(X, COEFFS_MUON, 5, restarts=[6])


@pytest.mark.parametrize("restarts", [[3, 5], [2, 4, 6], [4, 7]])
def test_shifted_gram_several_restarts_matches_scalar_model(restarts):
    """The scalar model of Appendix B.2.1 (-delta at every Gram formation) with
    several restarts: each restart sets x <- q x, r <- x^2 - delta, q <- 1."""
    delta = 4e-4
    T = 8
    rng = np.random.default_rng(33)
    X = oracle.normalize(rng.standard_normal((8, 24)) @ np.diag(np.logspace(0, -2, 24)), 1.0)
    U, S, Vt = np.linalg.svd(X, full_matrices=False)
    x = S.copy()
    r = x * x - delta
    q = np.ones_like(x)
    a, b, c = COEFFS_CLASSIC
    for t in range(1, T + 1):
        if t in restarts:
            x = q * x
            r = x * x - delta
            q = np.ones_like(x)
        z = a + b * r + c * r * r
        r = r * z * z
        q = q * z
    exp = (U * (q * x)[None, :]) @ Vt
    got = oracle.gram_ns(X, COEFFS_CLASSIC, T, gram_shift=delta, restarts=restarts)
    assert rel(got, exp) <= 1e-11


def test_naive_gram_diverges_with_spurious_negative_eigenvalue():
    """Appendix B.1.2: with h(x) = 15/8 - 10/8 x + 3/8 x^2, a negative
    eigenvalue of R grows by more than (15/8)^2 per step and diverges; the
    same iteration without the shift stays bounded."""
    rng = np.random.default_rng(13)
    # many tiny singular values, as for a Muon momentum: sigma^2 < 4e-4
    u, _ = np.linalg.qr(rng.standard_normal((16, 16)))
    v, _ = np.linalg.qr(rng.standard_normal((64, 16)))
    X = oracle.normalize((u * np.logspace(0, -3, 16)[None, :]) @ v.T, 1.0)
    with np.errstate(all="ignore"):
        bad = oracle.naive_gram_ns(X, COEFFS_CLASSIC, 10, r0_shift=4e-4)
    good = oracle.naive_gram_ns(X, COEFFS_CLASSIC, 10, r0_shift=0.0)
    assert (not np.all(np.isfinite(bad))) or np.abs(bad).max() > 1e6
    assert np.linalg.norm(good, 2) <= 1.0 + 1e-9
    # and the explicit-aI form equals the implicit one when unshifted
    assert rel(good, oracle.gram_ns(X, COEFFS_CLASSIC, 10, 0)) <= 1e-12


# --------------------------------------------------------------------------
# FLOP figures printed on the pages
# --------------------------------------------------------------------------

def test_flop_savings_match_printed_figures():
    cases = json.load(open(os.path.join(GOLDEN, "flop_savings.json")))["cases"]
    n = 1024
    for case in cases:
        T = case["T"]
        if "alpha" in case:
            m = case["alpha"] * n
            std = oracle.flops_standard(n, m, T)
            sym = oracle.flops_standard_symmetric(n, m, T)
            naive = oracle.flops_gram_naive(n, m, T)
            stable = oracle.flops_gram_stable(n, m, T)
            if "without symmetric" in case["what"]:
                saving = 1 - naive / std
            elif "stable" in case["what"]:
                saving = 1 - stable / sym
            else:
                saving = 1 - naive / sym
            assert round(100 * saving) == case["printed_percent"], case
        else:
            H = case["H"]
            d = 16 * 256
            big = oracle.flops_standard_symmetric(d, d, T)
            small = H * oracle.flops_gram_naive(d // H, d, T)
            ratio = big / small
            # printed as "80x"; the formulas give 20*256/65 = 78.8
            assert abs(ratio - case["printed_ratio"]) / case["printed_ratio"] < 0.02, ratio


def test_flop_formulas_closed_forms():
    """2T(2a+1) = 20a+10 at T=5 (Section 2.2); restart costs 3(a-1)n^3
    (Section 4.2); Gram equals symmetric standard at a = 1 (Section 4.1)."""
    n = 512
    for alpha in (1, 2, 4, 8):
        m = alpha * n
        assert oracle.flops_standard(n, m, 5) == (20 * alpha + 10) * n ** 3
        assert oracle.flops_gram_stable(n, m, 5) - oracle.flops_gram_naive(n, m, 5) \
            == 3 * (alpha - 1) * n ** 3
        assert oracle.flops_gram_stable(n, m, 5) == (4 * 5 + 6 * alpha - 6) * n ** 3
    assert oracle.flops_gram_naive(n, n, 5) == oracle.flops_standard_symmetric(n, n, 5)
