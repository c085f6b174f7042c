"""GPU test of the entry point that allocates nothing (ns_orthogonalize_noalloc):
through the C ABI, two calls in a row on the library's fixed scratch (the
second bucket smaller, so it runs over what the first left behind), each bit
for bit equal to ns_orthogonalize with a workspace of its own, and within the
oracle's bars."""
import ctypes

import numpy as np
import pytest
import torch

import newton_schulz_gram_amd as nsg
import oracle
from synth import COEFFS_MUON
from synth.workloads import custom

pytestmark = pytest.mark.gpu


def _noalloc(x, out, status, **kw):
    p, keep = nsg.make_params(**kw)
    G, R, C = x.shape
    code = nsg.lib().ns_orthogonalize_noalloc(
        ctypes.c_void_p(x.data_ptr()), nsg._dtype_code(x.dtype), ctypes.c_void_p(out.data_ptr()),
        nsg._dtype_code(out.dtype), G, R, C, ctypes.byref(p), ctypes.c_void_p(status.data_ptr()),
        ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert code == 0, nsg.STATUS.get(code, code)


def _with_workspace(x, **kw):
    p, keep = nsg.make_params(**kw)
    G, R, C = x.shape
    ws = torch.empty(max(1, nsg.workspace_size(G, R, C, **kw)), dtype=torch.uint8, device=x.device)
    out = torch.empty_like(x)
    code = nsg.lib().ns_orthogonalize(
        ctypes.c_void_p(x.data_ptr()), nsg._dtype_code(x.dtype), ctypes.c_void_p(out.data_ptr()),
        nsg._dtype_code(out.dtype), G, R, C, ctypes.byref(p), ctypes.c_void_p(ws.data_ptr()), ws.numel(), None,
        ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert code == 0
    return out


@pytest.mark.parametrize("kw", [dict(), dict(mode="standard"), dict(compute_dtype="bf16", restart_after=3)])
def test_noalloc_matches_workspace_entry_point(kw):
    first = custom(6, 700, 1800, "f16", "gaussian", seed=71).cuda()      # several tiles plus a ragged tail
    second = custom(2, 200, 520, "f16", "gaussian", seed=72).cuda()      # smaller: runs over stale scratch
    assert nsg.workspace_size(6, 700, 1800, **kw) <= nsg.NOALLOC_MAX_BYTES
    refs = [_with_workspace(x, **kw) for x in (first, second)]
    torch.cuda.synchronize()
    for x, ref in zip((first, second), refs):
        out = torch.full_like(x, float("nan"))
        st = torch.full((x.shape[0],), 7, dtype=torch.int32, device="cuda")
        _noalloc(x, out, st, **kw)
        torch.cuda.synchronize()
        assert torch.equal(out, ref)
        assert st.tolist() == [0] * x.shape[0]
        o = oracle.orthogonalize(x.double().cpu().numpy(), 5, COEFFS_MUON, kw.get("mode", "gram"),
                                 kw.get("restart_after", 2), 1.05)
        d = out.double().cpu().numpy() - o
        rel = np.linalg.norm(d.reshape(len(o), -1), axis=1) / np.linalg.norm(o.reshape(len(o), -1), axis=1)
        assert rel.max() <= 3e-2, rel


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_noalloc_with_the_input_read_in_place(dtype):
    """16-bit buckets whose sides are multiples of 256 are read in place by
    the products (no scaled copy in the scratch; a bf16 input under fp16
    compute through the raw R0 and the converting X = QX0, and one matrix of
    the first bucket, scaled by 2^-40, through the bf16 copy the scale pass
    writes into the scratch); two calls in a row, the second smaller, each bit
    for bit equal to the workspace entry point."""
    first = custom(4, 768, 2048, dtype, "gaussian", seed=74).cuda()   # wide, Gram
    second = custom(3, 2048, 512, dtype, "gaussian", seed=75).cuda()  # tall, Gram
    if dtype == "bf16":
        first[1] *= 2.0 ** -40
    for x in (first, second):
        assert [e["label"] for e in nsg.plan(x.shape[1], x.shape[2], in_dtype=dtype)][1] == "scales"
        assert nsg.workspace_size(*x.shape) <= nsg.NOALLOC_MAX_BYTES
    refs = [_with_workspace(x) for x in (first, second)]
    torch.cuda.synchronize()
    for x, ref in zip((first, second), refs):
        out = torch.full_like(x, float("nan"))
        st = torch.full((x.shape[0],), 7, dtype=torch.int32, device="cuda")
        _noalloc(x, out, st)
        torch.cuda.synchronize()
        assert torch.equal(out, ref)
        assert st.tolist() == [0] * x.shape[0]


def test_noalloc_binding_and_oversize():
    x = custom(3, 256, 1024, "bf16", "gaussian", seed=73).cuda()
    out = torch.empty_like(x)
    nsg.orthogonalize_noalloc(x, out)
    torch.cuda.synchronize()
    assert torch.equal(out, nsg.orthogonalize(x))
    big = torch.empty((64, 512, 4096), dtype=torch.float16, device="cuda")
    assert nsg.workspace_size(64, 512, 4096) > nsg.NOALLOC_MAX_BYTES
    with pytest.raises(nsg.NSGError) as e:
        nsg.orthogonalize_noalloc(big, torch.empty_like(big))
    assert e.value.code == 6
