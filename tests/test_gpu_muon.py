"""GPU tests of the Muon step (Dion3 paper, Eq. (1); Algorithm 4, steps 8-9;
the muon card's stochastic-rounding write-back) against the CPU oracle.

The momentum and update kernels are elementwise fp32 arithmetic with one
rounding per operation and Philox random bits, so they are compared bit for
bit; the whole step compares the orthogonalized part at the Newton-Schulz
tolerance."""
import numpy as np
import pytest
import torch

import newton_schulz_gram_amd as nsg
import oracle
from oracle import muon_oracle as mo
from synth.workloads import custom

pytestmark = pytest.mark.gpu

TDT = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}


def as_f32(t):
    return t.float().cpu().numpy()


def bits(t):
    return t.cpu().view(torch.int16).numpy().view(np.uint16)


@pytest.mark.parametrize("m_dt", ["f32", "bf16"])
@pytest.mark.parametrize("g_dt", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("n,off", [(4096, 0), (1001, 0), (4096, 3)])
def test_momentum_bitwise(m_dt, g_dt, n, off):
    rng = np.random.default_rng(n + off)
    m0 = torch.from_numpy(rng.standard_normal(n + off).astype(np.float32)).to(TDT[m_dt]).cuda()
    g0 = torch.from_numpy(rng.standard_normal(n + off).astype(np.float32)).to(TDT[g_dt]).cuda()
    M, G = m0[off:], g0[off:]
    ref = mo.momentum(as_f32(M), as_f32(G), 0.95)
    nsg.muon_momentum(M, G, 0.95)
    torch.cuda.synchronize()
    if m_dt == "f32":
        assert np.array_equal(M.cpu().numpy().view(np.uint32), ref.view(np.uint32))
    else:
        assert np.array_equal(bits(M), mo.bf16_bits_rne(ref))


@pytest.mark.parametrize("w_dt", ["f32", "bf16"])
@pytest.mark.parametrize("o_dt", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("stochastic", [True, False])
@pytest.mark.parametrize("n,off", [(65536, 0), (777, 0), (8192, 5)])
def test_update_bitwise(w_dt, o_dt, stochastic, n, off):
    rng = np.random.default_rng(7 * n + off)
    w0 = torch.from_numpy(rng.standard_normal(n + off).astype(np.float32)).to(TDT[w_dt]).cuda()
    o0 = torch.from_numpy(rng.standard_normal(n + off).astype(np.float32)).to(TDT[o_dt]).cuda()
    W, O = w0[off:], o0[off:]
    lr, wd, s, seed, step = 0.02, 0.1, 0.75, 123456789012345, 42
    if w_dt == "f32":
        ref = mo.update_f32(as_f32(W), as_f32(O), lr, wd, s)
    else:
        # the element index is the position within W (its global index)
        ref = mo.update_bf16(bits(W), as_f32(O), lr, wd, s, seed, step, stochastic)
    nsg.muon_update(W, O, lr, wd, s, stochastic=stochastic, seed=seed, step=step)
    torch.cuda.synchronize()
    if w_dt == "f32":
        assert np.array_equal(W.cpu().numpy().view(np.uint32), ref.view(np.uint32))
    else:
        assert np.array_equal(bits(W), ref)


def test_stochastic_rounding_unbiased_on_gpu():
    n = 200000
    W = torch.ones(n, dtype=torch.bfloat16, device="cuda")
    O = torch.ones(n, dtype=torch.float32, device="cuda")
    lr = 0.3 * 2.0 ** -8
    nsg.muon_update(W, O, lr, seed=5, step=1)
    Wn = torch.ones(n, dtype=torch.bfloat16, device="cuda")
    nsg.muon_update(Wn, O, lr, stochastic=False)
    torch.cuda.synchronize()
    exact = float(np.float32(1.0) - np.float32(lr))
    sigma = 2.0 ** -8 * np.sqrt(0.21 / n)
    assert abs(W.double().mean().item() - exact) <= 5 * sigma
    assert torch.all(Wn == 1.0)
    # same (seed, step): same bits; another step: different bits
    W2 = torch.ones(n, dtype=torch.bfloat16, device="cuda")
    nsg.muon_update(W2, O, lr, seed=5, step=1)
    W3 = torch.ones(n, dtype=torch.bfloat16, device="cuda")
    nsg.muon_update(W3, O, lr, seed=5, step=2)
    torch.cuda.synchronize()
    assert torch.equal(W, W2) and not torch.equal(W, W3)


@pytest.mark.parametrize("shape", [(3, 256, 1024), (2, 768, 300)])
def test_muon_step_matches_oracle(shape):
    G, R, C = shape
    rng = np.random.default_rng(9)
    W = torch.from_numpy(rng.standard_normal(shape).astype(np.float32)).cuda()
    M = torch.from_numpy(0.1 * rng.standard_normal(shape).astype(np.float32)).cuda()
    Gr = custom(G, R, C, "bf16", "gaussian", seed=81).cuda()
    W0, M0 = as_f32(W), as_f32(M)
    mu, lr, wd, s = 0.95, 0.02, 0.01, 0.5
    nsg.muon_step(W, M, Gr, mu, lr, wd, s)
    torch.cuda.synchronize()
    m_ref = mo.momentum(M0, as_f32(Gr), mu)
    assert np.array_equal(as_f32(M).view(np.uint32), m_ref.view(np.uint32))
    o_ref = oracle.orthogonalize(m_ref.astype(np.float64), 5, (3.4445, -4.7750, 2.0315), "gram", 2, 1.05)
    c1, c2 = np.float32(1 - lr * wd), np.float32(lr * s)
    o_gpu = (c1 * W0.astype(np.float64) - as_f32(W).astype(np.float64)) / np.float64(c2)
    for g in range(G):
        rel = np.linalg.norm(o_gpu[g] - o_ref[g]) / np.linalg.norm(o_ref[g])
        assert rel <= 3e-2, (g, rel)
