"""GPU parity of the Dion3 selection front-end (Dion3 paper, Section 6;
Algorithm 4, steps 3-4) against the CPU oracle, through the C ABI.

Index work is compared exactly: the GPU's fp64 l1 norms agree with the
oracle's exact sums to ~1e-15 relative, so the selected set is the oracle's
unless two norms at the selection boundary lie within that rounding; there
either choice is correct, and the test checks that the GPU's choice is valid.
"""
import math

import numpy as np
import pytest
import torch

import newton_schulz_gram_amd as nsg
import oracle
import synth
from synth import WORKLOADS
from synth.workloads import custom

pytestmark = pytest.mark.gpu

HALF_REL, HALF_COS = 3e-2, 0.97
NORM_REL = 1e-13


def check_selection(idx_gpu, M64, k, dim):
    """idx_gpu equals the oracle's selection, or differs only inside a
    near-tie at the boundary."""
    for g in range(M64.shape[0]):
        S, norms, kk, d = oracle.select(M64[g], 1.0, dim)  # norms only
        order = sorted(range(len(norms)), key=lambda i: (-norms[i], i))
        exp = sorted(order[:k])
        got = sorted(int(i) for i in idx_gpu[g])
        assert got == [int(i) for i in idx_gpu[g]], "indices not ascending"
        if got == exp:
            continue
        kth = norms[order[k - 1]]
        for i in set(got) ^ set(exp):
            assert abs(norms[i] - kth) <= 1e-12 * max(kth, 1e-300), (g, i)


@pytest.mark.parametrize("dtype", ["f16", "bf16", "f32"])
@pytest.mark.parametrize("dim", [0, 1])
@pytest.mark.parametrize("shape", [(3, 300, 1000), (2, 1000, 300), (1, 257, 513), (2, 64, 7)])
def test_l1_norms(dtype, dim, shape):
    G, R, C = shape
    x = custom(G, R, C, dtype, "gaussian", seed=51)
    keys = nsg.l1_norms(x.cuda(), dim).cpu().numpy()
    torch.cuda.synchronize()
    x64 = x.double().numpy()
    for g in range(G):
        ref = oracle.l1_norms(x64[g], dim)
        assert np.all(np.abs(keys[g] - ref) <= NORM_REL * ref + 1e-300), (g, np.max(np.abs(keys[g] - ref) / ref))


@pytest.mark.parametrize("n,k", [(1, 1), (10, 3), (1000, 1), (1000, 1000), (3000, 777), (5000, 1250), (65536, 8192)])
def test_topk_exact_with_ties(n, k):
    """Keys with many exact ties (integers), and the lower-index rule."""
    rng = np.random.default_rng(n + k)
    G = 3
    keys = rng.integers(0, max(2, n // 4), size=(G, n)).astype(np.float64)
    keys[1] = 5.0  # all equal: the first k indices
    idx, pos = nsg.topk(torch.from_numpy(keys).cuda(), k)
    idx, pos = idx.cpu().numpy(), pos.cpu().numpy()
    for g in range(G):
        order = sorted(range(n), key=lambda i: (-keys[g][i], i))
        exp = np.array(sorted(order[:k]))
        assert np.array_equal(idx[g], exp), g
        p = np.full(n, -1)
        p[exp] = np.arange(k)
        assert np.array_equal(pos[g], p)


def test_topk_real_keys():
    rng = np.random.default_rng(3)
    keys = np.abs(rng.standard_normal((4, 11008))) * 10.0 ** rng.uniform(-3, 3, size=(4, 11008))
    idx, _ = nsg.topk(torch.from_numpy(keys).cuda(), 2752)
    for g in range(4):
        exp = np.sort(np.argsort(-keys[g], kind="stable")[:2752])
        assert np.array_equal(idx[g].cpu().numpy(), exp)


@pytest.mark.parametrize("dim", [0, 1])
@pytest.mark.parametrize("shape,fraction", [((4, 768, 3072), 0.25), ((3, 3072, 768), 0.125), ((2, 300, 1000), 0.5),
                                            ((2, 1000, 300), 0.3)])
def test_orthogonalize_selected_matches_oracle(dim, shape, fraction):
    G, R, C = shape
    x = custom(G, R, C, "f16", "gaussian", seed=52)
    out, idx = nsg.orthogonalize_selected(x.cuda(), fraction, dim=dim)
    torch.cuda.synchronize()
    ref, S = oracle.select_orthogonalize(x.double().numpy(), fraction, dim=dim)
    n = R if dim == 0 else C
    k = oracle.n_selected(n, fraction)
    assert idx.shape == (G, k)
    idx = idx.cpu().numpy()
    check_selection(idx, x.double().numpy(), k, dim)
    o = out.double().cpu().numpy()
    for g in range(G):
        if not np.array_equal(idx[g], S[g]):
            continue  # near-tie at the boundary: the parity of O is not defined there
        a = o[g][S[g], :] if dim == 0 else o[g][:, S[g]]
        b = ref[g][S[g], :] if dim == 0 else ref[g][:, S[g]]
        rel = np.linalg.norm(a - b) / np.linalg.norm(b)
        cos = np.sum(a * b) / (np.linalg.norm(a) * np.linalg.norm(b))
        assert rel <= HALF_REL and cos >= HALF_COS, (g, rel, cos)
        mask = np.ones(n, dtype=bool)
        mask[S[g]] = False
        rest = o[g][mask, :] if dim == 0 else o[g][:, mask]
        assert not rest.any()


def test_default_dimension_and_7b_fraction_quarter():
    """11008 x 4096 bf16 (7B MLP): the smaller dimension is the columns;
    k = 1024 columns, submatrix 11008 x 1024 (alpha grows by 1/f)."""
    w = WORKLOADS["llama7b_mlp_32x11008x4096_bf16"]
    x = synth.make(w)[:2].contiguous()
    out, idx = nsg.orthogonalize_selected(x.cuda(), 0.25, safety=w.safety)
    torch.cuda.synchronize()
    assert idx.shape == (2, 1024) and out.shape == (2, 11008, 4096) and out.dtype == torch.bfloat16
    ref, S = oracle.select_orthogonalize(x[:1].double().numpy(), 0.25, safety=w.safety)
    check_selection(idx[:1].cpu().numpy(), x[:1].double().numpy(), 1024, 1)
    if np.array_equal(idx[0].cpu().numpy(), S[0]):
        a = out[0].double().cpu().numpy()[:, S[0]]
        b = ref[0][:, S[0]]
        assert np.linalg.norm(a - b) / np.linalg.norm(b) <= HALF_REL
    # grouped == single, bitwise
    one, i1 = nsg.orthogonalize_selected(x[1:2].cuda(), 0.25, safety=w.safety)
    assert torch.equal(one[0], out[1]) and torch.equal(i1[0], idx[1])


def test_fraction_one_equals_plain_call():
    """f = 1 selects every row in order: the result is ns_orthogonalize's,
    bit for bit (Section 6: f = 1 is Muon)."""
    x = custom(3, 256, 1024, "f16", "gaussian", seed=53).cuda()
    a, idx = nsg.orthogonalize_selected(x, 1.0, dim=0)
    b = nsg.orthogonalize(x)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    assert torch.equal(idx.cpu(), torch.arange(256, dtype=torch.int32).repeat(3, 1))


def test_selected_in_place():
    x = custom(2, 200, 800, "f16", "gaussian", seed=54).cuda()
    ref, _ = nsg.orthogonalize_selected(x.clone(), 0.25)
    out, _ = nsg.orthogonalize_selected(x, 0.25, out=x)
    torch.cuda.synchronize()
    assert torch.equal(out, ref) and out.data_ptr() == x.data_ptr()
