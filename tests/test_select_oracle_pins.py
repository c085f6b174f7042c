"""Pins of the selection front-end oracle (Dion3 paper, Section 6 and
Algorithm 4, steps 3-4) to facts outside its own code (CPU only)."""
import numpy as np
import pytest

import oracle
from synth import COEFFS_MUON


def svd_polar_ns(Y, steps=5, coeffs=COEFFS_MUON, safety=1.05, eps=oracle.EPS):
    """U p_T..p_1(sigma / (s (nu + eps))) V^T from LAPACK's SVD (Section 2.2)."""
    U, S, Vt = np.linalg.svd(Y, full_matrices=False)
    x = S / (safety * (np.sqrt(np.sum(S * S)) + eps))
    for _ in range(steps):
        a, b, c = coeffs
        x = a * x + b * x ** 3 + c * x ** 5
    return (U * x[None, :]) @ Vt


def test_k_is_ceil_f_n():
    assert oracle.n_selected(4096, 0.25) == 1024
    assert oracle.n_selected(4096, 1 / 8) == 512
    assert oracle.n_selected(10, 0.25) == 3
    assert oracle.n_selected(7, 1.0) == 7
    assert oracle.n_selected(3, 0.01) == 1
    with pytest.raises(ValueError):
        oracle.n_selected(10, 0.0)


def test_selects_largest_l1_rows_hand_built():
    """Rows with l1 norms 3, 10, 1, 7, 7, 2: the top 3 are rows 1, 3, 4; top 2
    breaks the 7/7 tie by the lower index (row 3)."""
    M = np.zeros((6, 4))
    for i, v in enumerate([3, 10, 1, 7, 7, 2]):
        M[i, i % 4] = -v if i % 2 else v  # l1 ignores the sign
    S, norms, k, d = oracle.select(M, 0.5, dim=0)
    assert d == 0 and k == 3 and list(S) == [1, 3, 4]
    assert list(norms) == [3, 10, 1, 7, 7, 2]
    S2, _, k2, _ = oracle.select(M, 2 / 6, dim=0)
    assert k2 == 2 and list(S2) == [1, 3]


def test_l1_norms_match_brute_force():
    rng = np.random.default_rng(5)
    M = rng.standard_normal((9, 33)).astype(np.float16).astype(np.float64)
    rows = oracle.l1_norms(M, 0)
    cols = oracle.l1_norms(M, 1)
    for i in range(9):
        assert rows[i] == sum(abs(float(v)) for v in M[i])
    for j in range(33):
        assert abs(cols[j] - sum(abs(float(v)) for v in M[:, j])) <= 1e-15 * cols[j]


@pytest.mark.parametrize("dim", [0, 1])
def test_output_is_polar_of_selected_submatrix(dim):
    rng = np.random.default_rng(6)
    M = rng.standard_normal((24, 40)) * np.logspace(0, -1, 40)[None, :]
    out, idx = oracle.select_orthogonalize(M[None], 0.25, dim=dim)
    S = idx[0]
    sub = M[S, :] if dim == 0 else M[:, S]
    exp = svd_polar_ns(sub)
    got = out[0][S, :] if dim == 0 else out[0][:, S]
    assert np.linalg.norm(got - exp) <= 1e-10 * np.linalg.norm(exp)
    mask = np.ones(M.shape[dim], dtype=bool)
    mask[S] = False
    rest = out[0][mask, :] if dim == 0 else out[0][:, mask]
    assert not rest.any()


def test_fraction_one_is_muon():
    """f = 1 selects everything: the update rule reduces to Muon (Section 6)."""
    rng = np.random.default_rng(7)
    M = rng.standard_normal((16, 48))
    out, idx = oracle.select_orthogonalize(M[None], 1.0, dim=0)
    assert list(idx[0]) == list(range(16))
    exp = svd_polar_ns(M)
    assert np.linalg.norm(out[0] - exp) <= 1e-10 * np.linalg.norm(exp)


def test_default_dimension_is_the_smaller_one():
    assert oracle.select_dim(100, 40) == 1 and oracle.select_dim(40, 100) == 0 and oracle.select_dim(50, 50) == 0
    rng = np.random.default_rng(8)
    M = rng.standard_normal((30, 12))
    a, ia = oracle.select_orthogonalize(M[None], 0.5)          # columns (12 < 30)
    b, ib = oracle.select_orthogonalize(M.T[None].copy(), 0.5, dim=0)
    assert np.array_equal(ia, ib)
    assert np.linalg.norm(a[0] - b[0].T) <= 1e-12 * np.linalg.norm(a[0])
