"""Plain fp64 CPU oracle for the Dion3 selection front-end.

TEST INFRASTRUCTURE ONLY (like ns_oracle): used by the tests, never by the
product path; shares no code with the HIP library.

Dion3 paper, Section 6 ("Selection", "Orthogonalization") and Algorithm 4,
steps 3-4:
    S <- indices of the k = ceil(f n) rows of M with the largest l1 norm
    O <- polar(M[S, :])             (the k x m submatrix, by Newton-Schulz)
Rows may be replaced by columns; without sharding the pages select along the
smaller dimension.  The update and error-feedback steps (5-10) are not part
of this front-end.

Readings of points the pages leave open:
  * the l1 norms are exact sums of |M_ij| (math.fsum, correctly rounded), so
    the selection is fixed by the data alone;
  * equal norms are broken by the lower index; S is kept in ascending order
    (polar commutes with permuting rows, so the order only fixes the layout);
  * the result is scattered back into an R x C array with zeros in the rows
    (columns) that were not selected, and S is returned alongside.
"""
from __future__ import annotations

import math

import numpy as np

from .ns_oracle import ns_matrix


def n_selected(n: int, fraction: float) -> int:
    """k = ceil(f n), at least 1 for n >= 1 (Algorithm 4, step 3)."""
    if not 0.0 < fraction <= 1.0:
        raise ValueError("fraction must lie in (0, 1]")
    return min(n, max(1, math.ceil(fraction * n))) if n else 0


def select_dim(R: int, C: int, dim: int = -1) -> int:
    """0: rows, 1: columns; -1 picks the smaller dimension (rows on a tie)."""
    if dim in (0, 1):
        return dim
    return 1 if C < R else 0


def l1_norms(M: np.ndarray, dim: int) -> np.ndarray:
    """Exact l1 norm of every row (dim 0) or column (dim 1)."""
    A = np.abs(np.asarray(M, dtype=np.float64))
    lines = A if dim == 0 else A.T
    return np.array([math.fsum(line) for line in lines], dtype=np.float64)


def select(M: np.ndarray, fraction: float, dim: int = -1):
    """(S ascending, the norms, k, dim) for one R x C matrix."""
    R, C = M.shape
    d = select_dim(R, C, dim)
    n = R if d == 0 else C
    k = n_selected(n, fraction)
    norms = l1_norms(M, d)
    # largest norm first, lower index first among equals
    order = sorted(range(n), key=lambda i: (-norms[i], i))
    S = np.array(sorted(order[:k]), dtype=np.int64)
    return S, norms, k, d


def select_orthogonalize(Ms: np.ndarray, fraction: float, dim: int = -1, steps: int = 5,
                         coeffs=(3.4445, -4.7750, 2.0315), mode: str = "gram",
                         restart_after: int = 2, safety: float = 1.05, restarts=None):
    """Bucket [G, R, C] -> (out [G, R, C] with polar(M[S]) in the selected rows
    or columns and zeros elsewhere, S [G, k])."""
    Ms = np.asarray(Ms, dtype=np.float64)
    G, R, C = Ms.shape
    out = np.zeros_like(Ms)
    idx = []
    for g in range(G):
        S, _, _, d = select(Ms[g], fraction, dim)
        sub = Ms[g][S, :] if d == 0 else Ms[g][:, S]
        O = ns_matrix(sub, steps, coeffs, mode, restart_after, safety, restarts=restarts)
        if d == 0:
            out[g][S, :] = O
        else:
            out[g][:, S] = O
        idx.append(S)
    return out, np.stack(idx) if idx else np.zeros((0, 0), dtype=np.int64)
