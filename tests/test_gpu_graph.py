"""HIP-graph capture of a whole call (Dion3 paper, Section 7: the launch
sequence is the same every step, so it is captured once and replayed).

Every replay is checked against the eager result, bit for bit, with eager
work and synchronisations between the replays.
"""
import pytest
import torch

import newton_schulz_gram_amd as nsg
from synth.workloads import custom

pytestmark = pytest.mark.gpu


def _replays_match(fn, ref, x, fresh, n=4):
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        out = fn()
    for i in range(n):
        x.copy_(fresh[i % len(fresh)])
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        exp = ref(fresh[i % len(fresh)])
        got = out if not isinstance(out, tuple) else out[0]
        assert torch.equal(got, exp), i
        torch.matmul(torch.randn(64, 64, device="cuda"), torch.randn(64, 64, device="cuda"))  # eager work between


@pytest.mark.parametrize("shape,dtype", [((1, 128, 512), "f16"), ((4, 768, 3072), "f16"), ((8, 2048, 512), "f16"),
                                         ((4, 768, 3072), "bf16"), ((8, 2048, 512), "bf16")])
def test_graph_replay_orthogonalize(shape, dtype):
    """fp16 inputs read in place; bf16 ones (fp16 compute) read in place
    through the raw R0 and the converting X = QX0."""
    G, R, C = shape
    fresh = [custom(G, R, C, dtype, "gaussian", seed=60 + i).cuda() for i in range(2)]
    x = fresh[0].clone()
    out = torch.empty_like(x)
    ws = torch.empty(nsg.workspace_size(G, R, C), dtype=torch.uint8, device="cuda")
    st = torch.zeros(G, dtype=torch.int32, device="cuda")

    def fn():
        return nsg.orthogonalize(x, out=out, workspace=ws, status=st)

    _replays_match(fn, lambda v: nsg.orthogonalize(v), x, fresh)


def test_graph_replay_selected():
    fresh = [custom(4, 768, 3072, "bf16", "gaussian", seed=70 + i).cuda() for i in range(2)]
    x = fresh[0].clone()

    def fn():
        return nsg.orthogonalize_selected(x, 0.25)

    _replays_match(fn, lambda v: nsg.orthogonalize_selected(v, 0.25)[0], x, fresh)
