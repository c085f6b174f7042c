"""Pins of the Muon-step oracle (CPU only): the Philox known-answer vectors,
round-to-nearest-even against torch's conversion, and the defining properties
of stochastic rounding (the muon card, "Correctness": unbiased, sub-ULP
updates accumulate; round-to-nearest leaves them unchanged)."""
import json
import os

import numpy as np
import pytest
import torch

from oracle import muon_oracle as mo

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "philox4x32_10_kat.json")


def test_philox_known_answers():
    for case in json.load(open(GOLDEN))["cases"]:
        ctr = [int(v, 16) for v in case["ctr"]]
        key = [int(v, 16) for v in case["key"]]
        out = [int(v) for v in mo.philox4x32_10(ctr, key)]
        assert out == [int(v, 16) for v in case["out"]]


def test_rne_matches_torch():
    rng = np.random.default_rng(1)
    x = (rng.standard_normal(100000) * 10.0 ** rng.uniform(-30, 30, 100000)).astype(np.float32)
    x[:4] = [np.inf, -np.inf, 0.0, -0.0]
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(mo.bf16_bits_rne(x), ref)


def test_stochastic_rounding_neighbours_and_exact_values():
    rng = np.random.default_rng(2)
    x = (rng.standard_normal(50000) * 3).astype(np.float32)
    r = mo.sr_bits(x.size, seed=7, step=3)
    b = mo.bf16_bits_stochastic(x, r)
    y = mo.bf16_from_bits(b)
    lo = mo.bf16_from_bits((x.view(np.uint32) >> 16).astype(np.uint16))  # truncated magnitude
    hi = mo.bf16_from_bits(((x.view(np.uint32) >> 16) + 1).astype(np.uint16))
    assert np.all((y == lo) | (y == hi))
    exact = mo.bf16_from_bits(mo.bf16_bits_rne(x))
    assert np.array_equal(mo.bf16_bits_stochastic(exact, r), mo.bf16_bits_rne(exact))


def test_stochastic_rounding_is_unbiased():
    """A sub-ULP update of 200k bf16 ones: the mean of the stochastically
    rounded results is the exact value; round-to-nearest leaves 1.0."""
    n = 200000
    w = np.full(n, 0x3F80, dtype=np.uint16)  # bf16 1.0
    o = np.full(n, 1.0, dtype=np.float32)
    lr = 0.3 * 2.0 ** -8                     # 0.3 ULP below 1.0 (ULP of [0.5, 1) = 2^-8)
    exact = np.float64(np.float32(1.0) - np.float32(lr))
    sr = mo.bf16_from_bits(mo.update_bf16(w, o, lr, 0.0, 1.0, seed=11, step=5)).astype(np.float64)
    rn = mo.bf16_from_bits(mo.update_bf16(w, o, lr, 0.0, 1.0, seed=11, step=5, stochastic=False))
    ulp = 2.0 ** -8
    sigma = ulp * np.sqrt(0.3 * 0.7 / n)
    assert abs(sr.mean() - exact) <= 5 * sigma
    assert np.all(rn == 1.0)


def test_random_bits_depend_on_seed_step_and_index():
    a = mo.sr_bits(64, 1, 1)
    assert not np.array_equal(a, mo.sr_bits(64, 2, 1))
    assert not np.array_equal(a, mo.sr_bits(64, 1, 2))
    assert np.array_equal(a[16:], mo.sr_bits(48, 1, 1, start=16))
    # uniform 16-bit values: mean ~ 32767.5
    big = mo.sr_bits(400000, 5, 9)
    assert abs(big.mean() - 32767.5) < 300


def test_update_and_momentum_formulas():
    rng = np.random.default_rng(3)
    w = rng.standard_normal(1000).astype(np.float32)
    o = rng.standard_normal(1000).astype(np.float32)
    got = mo.update_f32(w, o, 0.02, 0.1, 0.5)
    exp = (1 - 0.02 * 0.1) * w.astype(np.float64) - 0.02 * 0.5 * o
    assert np.max(np.abs(got - exp)) <= 4e-7 * np.max(np.abs(exp))
    m = rng.standard_normal(1000).astype(np.float32)
    g = rng.standard_normal(1000).astype(np.float32)
    assert np.max(np.abs(mo.momentum(m, g, 0.95) - (0.95 * m.astype(np.float64) + g))) <= 1e-6
