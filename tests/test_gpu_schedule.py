"""GPU tests of the kernel's scheduling state.

The kernel runs one workgroup per compute unit, and the workgroups take work items from
atomic counters in a ring of slots in static device memory; every launch must leave its
slot at zero. These tests check that results stay bit-identical when the ring wraps
many times, when two streams run the kernel at once, and when the call is captured into
a graph and replayed between eager calls.
"""
import pytest
import torch

import block_sparse_attention_radial_amd as radial

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    radial.lib()


def problem(seed, heads=8, frames=8, tokens=1024, w0=512, d=64):
    g = torch.Generator(device="cuda").manual_seed(seed)
    n = frames * tokens
    q, k, v = (torch.randn(1, heads, n, d, generator=g, device="cuda").to(torch.bfloat16)
               for _ in range(3))
    mask = radial.build_mask(frames, tokens, w0).to("cuda")
    return q, k, v, mask


def test_counter_ring_wraps_many_times():
    """600 calls: every slot of the ring is used more than twice."""
    q, k, v, mask = problem(1)
    first = radial.attn_fwd(q, k, v, mask)
    out = torch.empty_like(first)
    for i in range(600):
        radial.attn_fwd(q, k, v, mask, out=out)
        if i % 100 == 99:
            torch.cuda.synchronize()
            assert torch.equal(out, first), i
    torch.cuda.synchronize()
    assert torch.equal(out, first)


def test_two_streams_at_once():
    """Two problems launched alternately on two streams, with no ordering between them."""
    a = problem(2)
    b = problem(3, heads=4, frames=6, tokens=1560, w0=1560, d=128)
    ref_a = radial.attn_fwd(*a)
    ref_b = radial.attn_fwd(*b)
    torch.cuda.synchronize()
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    outs_a = [torch.empty_like(ref_a) for _ in range(8)]
    outs_b = [torch.empty_like(ref_b) for _ in range(8)]
    for i in range(8):
        with torch.cuda.stream(sa):
            radial.attn_fwd(*a, out=outs_a[i])
        with torch.cuda.stream(sb):
            radial.attn_fwd(*b, out=outs_b[i])
    torch.cuda.synchronize()
    for i in range(8):
        assert torch.equal(outs_a[i], ref_a), ("a", i)
        assert torch.equal(outs_b[i], ref_b), ("b", i)


def test_graph_capture_and_replay():
    """A captured call replays bit-identically, with eager calls on other inputs in
    between and enough of them to wrap the eager part of the ring."""
    q, k, v, mask = problem(4)
    q2, k2, v2, _ = problem(5)
    ref = radial.attn_fwd(q, k, v, mask)
    ref2 = radial.attn_fwd(q2, k2, v2, mask)
    torch.cuda.synchronize()
    out = torch.empty_like(ref)
    out2 = torch.empty_like(ref2)
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        radial.attn_fwd(q, k, v, mask, out=out)  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        radial.attn_fwd(q, k, v, mask, out=out)
    for r in range(5):
        out.zero_()
        graph.replay()
        for _ in range(40):
            radial.attn_fwd(q2, k2, v2, mask, out=out2)
        torch.cuda.synchronize()
        assert torch.equal(out, ref), r
        assert torch.equal(out2, ref2), r
