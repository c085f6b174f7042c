"""CPU tests of the restart-schedule sweep tool (Dion3 paper, Appendix B.2.1),
pinned against the oracle on diagonal inputs and against the pages' scalar
statements."""
import math

import numpy as np
import pytest

import oracle
from newton_schulz_gram_amd import restart_sweep as rsw
from synth import COEFFS_CLASSIC, COEFFS_MUON


@pytest.mark.parametrize("steps,restarts", [(5, []), (5, [3]), (8, [3, 5]), (6, [2, 4, 6])])
def test_scalar_model_matches_oracle_on_diagonal_input(steps, restarts):
    """A diagonal X (singular vectors = coordinate axes): the oracle's shifted
    Gram iteration returns diag(x_T), which the sweep's scalar model must
    reproduce direction by direction."""
    delta = 4e-4
    x0 = np.array([0.0, 1e-3, 0.01, 0.05, 0.2, 0.5, 0.8, 1.0])
    X = np.zeros((8, 20))
    X[np.arange(8), np.arange(8)] = x0
    coeffs = list(COEFFS_CLASSIC) * steps
    got = oracle.gram_ns(X, coeffs, steps, gram_shift=delta, restarts=restarts)
    model = rsw.simulate(coeffs, steps, restarts, delta, x0=x0)["x_T"]
    assert np.allclose(np.diag(got[:, :8]), model, rtol=1e-12, atol=1e-14)


def test_no_shift_is_the_composed_polynomial():
    x0 = np.linspace(0.0, 1.0, 41)
    for restarts in ([], [2], [3, 4]):
        m = rsw.simulate(COEFFS_MUON, 5, restarts, delta=0.0, x0=x0)["x_T"]
        assert np.allclose(m, oracle.composed_polynomial(x0, COEFFS_MUON, 5), rtol=1e-12, atol=1e-14)


def test_negative_eigenvalue_grows_faster_than_h0_squared():
    """Appendix B.1.2: with h(x) = 15/8 - 10/8 x + 3/8 x^2 a negative
    eigenvalue of R is multiplied by more than (15/8)^2 every step."""
    s = rsw.simulate(COEFFS_CLASSIC, 8, [], delta=4e-4)
    r = s["min_r"]
    assert r[0] < 0
    for a, b in zip(r, r[1:]):
        assert b < a * (15 / 8) ** 2


def test_restarts_bound_q():
    """Restarting resets Q to I: with a restart every two steps the worst
    kappa(Q_t) stays small, without restarts it grows without bound."""
    no = rsw.simulate(COEFFS_MUON, 10, [], 4e-4)
    yes = rsw.simulate(COEFFS_MUON, 10, [3, 5, 7, 9], 4e-4)
    assert max(yes["kappa_q"]) < 100 < max(no["kappa_q"])


def test_sweep_enumerates_every_schedule():
    rows = rsw.sweep(COEFFS_MUON, 5, 1)
    assert sorted(tuple(r["restarts"]) for r in rows) == [(2,), (3,), (4,), (5,)]
    assert rows[0]["max_kappa_q"] <= rows[-1]["max_kappa_q"]
    assert len(rsw.sweep(COEFFS_MUON, 8, 2)) == math.comb(7, 2)
    with pytest.raises(ValueError):
        rsw.simulate(COEFFS_MUON, 5, [1])
