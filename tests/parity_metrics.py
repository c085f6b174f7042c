"""Error measures of a GPU result against the fp64 oracle, shared by the GPU
parity tests and the bench's parity sample.

Per matrix (o = GPU output, r = oracle output, both as float64):
  rel        ||o - r||_F / ||r||_F              (the pages' relative error)
  cos        <o, r> / (||o||_F ||r||_F)         (the muon card's cosine)
  block_rel  max over 256 x 256 blocks b of rms(o_b - r_b) / rms(r): the
             worst block's error against the matrix's typical entry, so one
             wrong tile (or a corner of one) stands out even where it barely
             moves the whole-matrix norm (a ragged edge block counts its own
             elements only)
  elem_max   max |o - r| / rms(r): a single wrong element

The bars the tests hold these to are in tests/test_gpu_parity.py.
"""
from __future__ import annotations

import numpy as np

BLOCK = 256


def _as_f64(x) -> np.ndarray:
    if hasattr(x, "detach"):
        x = x.detach().double().cpu().numpy()
    return np.asarray(x, dtype=np.float64)


def matrix_errors(o, r, block: int = BLOCK) -> dict:
    """The four measures for one R x C matrix."""
    o = _as_f64(o)
    r = _as_f64(r)
    d = o - r
    rn = np.linalg.norm(r)
    on = np.linalg.norm(o)
    rms = rn / np.sqrt(r.size) if r.size else 0.0
    R, C = r.shape
    worst = 0.0
    for i in range(0, R, block):
        for j in range(0, C, block):
            db = d[i:i + block, j:j + block]
            worst = max(worst, float(np.sqrt(np.mean(db * db))))
    tiny = 1e-300
    return {
        "rel": float(np.linalg.norm(d) / max(rn, tiny)),
        "cos": float(np.sum(o * r) / max(on * rn, tiny)),
        "block_rel": worst / max(rms, tiny),
        "elem_max": float(np.max(np.abs(d))) / max(rms, tiny) if d.size else 0.0,
    }


def bucket_errors(out, ref) -> list:
    """matrix_errors for every matrix of [G, R, C] results."""
    o = _as_f64(out)
    r = _as_f64(ref)
    return [matrix_errors(o[g], r[g]) for g in range(o.shape[0])]


def summary(errs: list) -> dict:
    """Worst case of each measure over a list of matrix_errors results."""
    if not errs:
        return {"n": 0}
    return {
        "n": len(errs),
        "rel_max": max(e["rel"] for e in errs),
        "cos_min": min(e["cos"] for e in errs),
        "block_rel_max": max(e["block_rel"] for e in errs),
        "elem_max": max(e["elem_max"] for e in errs),
    }
