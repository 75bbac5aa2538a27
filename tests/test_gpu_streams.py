"""Library calls captured in a HIP graph and issued on concurrent streams.

Each entry point only enqueues kernels on the caller's stream and allocates
nothing, so it can be captured (torch.cuda.graph) and replayed, and calls on two
streams can overlap.  Graph replays are compared bit for bit with the eager
result, several times, with eager work and synchronisations between replays.
"""

import pytest
import torch

from exact_attention_35_amd import api, inputs
from gpu_util import announce, dev

pytestmark = pytest.mark.gpu

BF = torch.bfloat16


def _inputs(seed, B=2, H=4, N=700, d=128):
    q, k, v, do = inputs.random_case(seed, B, H, N, d, "bf16", backward=True)
    return dev(q, BF), dev(k, BF), dev(v, BF), dev(do, BF)


def test_graph_capture_forward_backward():
    announce("graph capture fwd + bwd")
    tq, tk, tv, tdo = _inputs(61)
    # eager reference
    o_ref, lse_ref = api.forward(tq, tk, tv, None, True)
    g_ref = api.backward(tq, tk, tv, o_ref, lse_ref, tdo, None, True)
    torch.cuda.synchronize()
    # static buffers for the captured calls
    o = torch.empty_like(tq)
    lse = torch.empty_like(lse_ref)
    ws = torch.empty(api.bwd_workspace_size(*tq.shape), dtype=torch.uint8, device=tq.device)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up on the capture stream
        api.forward(tq, tk, tv, None, True, out=o, lse_out=lse)
        api.backward(tq, tk, tv, o, lse, tdo, None, True, workspace=ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        api.forward(tq, tk, tv, None, True, out=o, lse_out=lse)
        grads = api.backward(tq, tk, tv, o, lse, tdo, None, True, workspace=ws)
    for rep in range(4):
        o.zero_()
        for g in grads:
            g.zero_()
        _ = (tq.float() * 2.0).sum()  # unrelated eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref) and torch.equal(lse, lse_ref), rep
        for g, r in zip(grads, g_ref):
            assert torch.equal(g, r), rep


def test_concurrent_streams():
    """Two independent problems on two streams at once give the results each gives alone."""
    announce("concurrent streams")
    a = _inputs(62)
    b = _inputs(63, B=1, H=8, N=1500, d=64)
    ref_a = api.forward(*a[:3], None, True)
    ref_b = api.forward(*b[:3], None, False)
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    s1.wait_stream(torch.cuda.current_stream())
    s2.wait_stream(torch.cuda.current_stream())
    outs = []
    for _ in range(3):
        with torch.cuda.stream(s1):
            ra = api.forward(*a[:3], None, True)
        with torch.cuda.stream(s2):
            rb = api.forward(*b[:3], None, False)
        outs.append((ra, rb))
    torch.cuda.synchronize()
    for ra, rb in outs:
        assert torch.equal(ra[0], ref_a[0]) and torch.equal(ra[1], ref_a[1])
        assert torch.equal(rb[0], ref_b[0]) and torch.equal(rb[1], ref_b[1])
