"""Plain CPU oracle for the Muon step around the orthogonalization.

TEST INFRASTRUCTURE ONLY (like ns_oracle): used by the tests, never by the
product path; shares no code with the HIP library.

Dion3 paper, Section 2.1, Eq. (1) (Muon) and Algorithm 4, steps 8-9; the
"muon" kernel card ("How it works", "Correctness"):
    M <- mu M + G
    O  = NS(M)                              (ns_oracle)
    W <- (1 - lr wd) W - lr s O             (decoupled weight decay, scaled update)
with a bf16 W written back by stochastic rounding keyed by the element's
global index, so the expected value is exact and sub-ULP updates accumulate.

Arithmetic, fixed so that the GPU and this oracle round identically (they are
compared bit for bit): every operation is one fp32 operation rounded to
nearest even, with no fused multiply-add:
    momentum: t = f32(mu) * m ; m' = t + g
    update:   c1 = f32(1 - lr wd), c2 = f32(lr s) (host, from float64)
              t1 = c1 * w ; t2 = c2 * o ; w' = t1 - t2
Stochastic rounding of a finite fp32 value to bf16: add 16 random bits to the
fp32 bit pattern and truncate the low 16 bits (rounds the magnitude up with
probability equal to the discarded fraction); non-finite values round to
nearest even.  Random bits: Philox-4x32-10 (Salmon, Moraes, Dror, Shaw,
"Parallel random numbers: as easy as 1, 2, 3", SC 2011), key = the 64-bit
seed, counter = (i >> 3 as 64 bits, step as 64 bits) for element i; element i
uses the 16-bit half (i & 1) of output word (i & 7) >> 1.
"""
from __future__ import annotations

import numpy as np

M0, M1 = 0xD2511F53, 0xCD9E8D57      # Philox-4x32 multipliers
W0, W1 = 0x9E3779B9, 0xBB67AE85      # Weyl key increments
MASK32 = 0xFFFFFFFF


def philox4x32_10(ctr, key):
    """Philox-4x32 with 10 rounds on arrays: ctr (..., 4) uint32, key (..., 2)
    uint32 -> (..., 4) uint32."""
    c = np.asarray(ctr, dtype=np.uint64) & MASK32
    k = np.asarray(key, dtype=np.uint64) & MASK32
    x0, x1, x2, x3 = c[..., 0], c[..., 1], c[..., 2], c[..., 3]
    k0, k1 = k[..., 0], k[..., 1]
    for r in range(10):
        if r:
            k0 = (k0 + W0) & MASK32
            k1 = (k1 + W1) & MASK32
        p0 = np.uint64(M0) * x0
        p1 = np.uint64(M1) * x2
        hi0, lo0 = p0 >> np.uint64(32), p0 & np.uint64(MASK32)
        hi1, lo1 = p1 >> np.uint64(32), p1 & np.uint64(MASK32)
        x0, x1, x2, x3 = hi1 ^ x1 ^ k0, lo1, hi0 ^ x3 ^ k1, lo0
    return np.stack([x0, x1, x2, x3], axis=-1).astype(np.uint32)


def sr_bits(n: int, seed: int, step: int, start: int = 0) -> np.ndarray:
    """16 random bits for elements start .. start+n-1."""
    i = np.arange(start, start + n, dtype=np.uint64)
    grp = i >> np.uint64(3)
    ctr = np.stack([grp & np.uint64(MASK32), grp >> np.uint64(32),
                    np.full_like(grp, step & MASK32), np.full_like(grp, (step >> 32) & MASK32)], axis=-1)
    key = np.array([seed & MASK32, (seed >> 32) & MASK32], dtype=np.uint64)
    out = philox4x32_10(ctr, np.broadcast_to(key, ctr.shape[:-1] + (2,)))
    word = out[np.arange(n), ((i & np.uint64(7)) >> np.uint64(1)).astype(np.int64)].astype(np.uint64)
    half = (i & np.uint64(1))
    return ((word >> (half * np.uint64(16))) & np.uint64(0xFFFF)).astype(np.uint32)


def bf16_bits_rne(x32: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns, round to nearest even (NaN stays NaN)."""
    u = np.asarray(x32, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = ((u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)).astype(np.uint32)
    nan = np.isnan(np.asarray(x32, dtype=np.float32))
    r[nan] = ((u[nan] >> np.uint64(16)) | np.uint64(0x40)).astype(np.uint32)
    return (r & 0xFFFF).astype(np.uint16)


def bf16_bits_stochastic(x32: np.ndarray, r16: np.ndarray) -> np.ndarray:
    x32 = np.asarray(x32, dtype=np.float32)
    u = x32.view(np.uint32).astype(np.uint64)
    sr = ((u + np.asarray(r16, dtype=np.uint64)) >> np.uint64(16)).astype(np.uint32) & 0xFFFF
    fin = np.isfinite(x32)
    out = bf16_bits_rne(x32).astype(np.uint32)
    out[fin] = sr[fin]
    return out.astype(np.uint16)


def bf16_from_bits(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint32) << 16).view(np.float32)


def momentum(m: np.ndarray, g: np.ndarray, mu: float) -> np.ndarray:
    """M <- mu M + G in fp32 (two roundings); inputs as float32 arrays."""
    t = np.float32(mu) * np.asarray(m, dtype=np.float32)
    return (t + np.asarray(g, dtype=np.float32)).astype(np.float32)


def update_f32(w: np.ndarray, o: np.ndarray, lr: float, wd: float, scale: float) -> np.ndarray:
    c1 = np.float32(1.0 - lr * wd)
    c2 = np.float32(lr * scale)
    t1 = c1 * np.asarray(w, dtype=np.float32)
    t2 = c2 * np.asarray(o, dtype=np.float32)
    return (t1 - t2).astype(np.float32)


def update_bf16(w_bits: np.ndarray, o: np.ndarray, lr: float, wd: float, scale: float, seed: int, step: int,
                stochastic: bool = True) -> np.ndarray:
    """bf16 W (as bit patterns, flat) updated and written back; returns bits."""
    w = bf16_from_bits(w_bits.reshape(-1))
    v = update_f32(w, np.asarray(o, dtype=np.float32).reshape(-1), lr, wd, scale)
    if stochastic:
        return bf16_bits_stochastic(v, sr_bits(v.size, seed, step))
    return bf16_bits_rne(v)
