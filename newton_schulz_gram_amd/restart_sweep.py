"""Restart-schedule sweep for Gram Newton–Schulz (host-side planning tool).

Dion3 paper, Appendix B.2.1 ("When to Restart"): with a fixed number of
restarts, simulate the iteration in full precision for every possible restart
schedule, with a spurious eigenvalue injected each time a Gram matrix is
formed, and keep the schedule whose Q_t has the smallest worst condition
number over the steps.

Model (every matrix of the iteration shares the left singular vectors of X0,
so each direction evolves on its own, Theorem 2): a direction with singular
value x of the current X has Gram eigenvalue r = x^2 - delta (delta = 4e-4 in
the paper, the most negative spurious eigenvalue it observed), and q = 1.  At
step t, z = a_t + b_t r + c_t r^2, r <- r z^2, q <- q z.  A restart at the top
of step t sets x <- q x, r <- x^2 - delta, q <- 1.  The directions are x = 0
(a numerically null singular value: r = -delta, the dangerous case) and a
geometric grid of x in [1e-4, 1].

This does not run on the GPU and is not part of ns_orthogonalize; its output
is a value for `restart_after` or the `restarts` list.

    python -m newton_schulz_gram_amd.restart_sweep --steps 5 --restarts 1
"""
from __future__ import annotations

import argparse
import itertools
import json
from typing import Iterable, Optional, Sequence

import numpy as np

MUON = (3.4445, -4.7750, 2.0315)
DELTA = 4e-4


def _triples(coeffs: Sequence[float], steps: int):
    c = [float(v) for v in coeffs]
    if len(c) == 3:
        return [tuple(c)] * steps
    if len(c) != 3 * steps:
        raise ValueError("coeffs must hold 3 or 3*steps values")
    return [tuple(c[3 * i:3 * i + 3]) for i in range(steps)]


def directions(n_grid: int = 400) -> np.ndarray:
    """Singular values tracked: 0 and a geometric grid of [1e-4, 1]."""
    return np.concatenate([[0.0], np.geomspace(1e-4, 1.0, n_grid)])


def simulate(coeffs: Sequence[float], steps: int, restarts: Iterable[int] = (),
             delta: float = DELTA, x0: Optional[np.ndarray] = None):
    """Per-step extremes of the scalar model for one restart schedule.

    Returns a dict with, for t = 1..steps: min_r (smallest eigenvalue of R_t),
    max_q, kappa_q (max |q| / min |q| over the directions), and x_T (the
    final singular values q_T x, one per direction)."""
    rs = set(int(t) for t in restarts)
    if any(t < 2 or t > steps for t in rs):
        raise ValueError("restart steps must lie in 2..steps")
    x = directions() if x0 is None else np.asarray(x0, dtype=np.float64).copy()
    r = x * x - delta
    q = np.ones_like(x)
    min_r, max_q, kappa = [], [], []
    with np.errstate(over="ignore", invalid="ignore"):
        for t, (a, b, c) in enumerate(_triples(coeffs, steps), start=1):
            if t in rs:
                x = q * x
                r = x * x - delta
                q = np.ones_like(x)
            z = a + b * r + c * r * r
            r = r * z * z
            q = q * z
            aq = np.abs(q)
            min_r.append(float(np.min(r)))
            max_q.append(float(np.max(aq)))
            kappa.append(float(np.max(aq) / np.min(aq)))
        x_T = q * x
    return {"min_r": min_r, "max_q": max_q, "kappa_q": kappa, "x_T": x_T}


def sweep(coeffs: Sequence[float] = MUON, steps: int = 5, n_restarts: int = 1,
          delta: float = DELTA):
    """Every schedule of `n_restarts` restart steps in 2..steps, best first
    (smallest worst kappa(Q_t), then largest worst min eigenvalue of R_t)."""
    out = []
    for sched in itertools.combinations(range(2, steps + 1), n_restarts):
        s = simulate(coeffs, steps, sched, delta)
        worst_k = max(s["kappa_q"])
        worst_k = worst_k if np.isfinite(worst_k) else float("inf")
        out.append({"restarts": list(sched), "restart_after": [t - 1 for t in sched],
                    "max_kappa_q": worst_k, "min_r": min(s["min_r"]), "max_q": max(s["max_q"])})
    out.sort(key=lambda d: (d["max_kappa_q"], -d["min_r"]))
    return out


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--restarts", type=int, default=1, help="number of restarts")
    ap.add_argument("--coeffs", type=float, nargs="+", default=list(MUON),
                    help="3 values, or 3 per step")
    ap.add_argument("--delta", type=float, default=DELTA)
    a = ap.parse_args(argv)
    for row in sweep(a.coeffs, a.steps, a.restarts, a.delta):
        print(json.dumps(row))


if __name__ == "__main__":
    main()
