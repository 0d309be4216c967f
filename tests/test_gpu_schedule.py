"""GPU tests of the kernel's scheduling state.

The kernel runs one workgroup per compute unit, and the workgroups take work items from
atomic counters in a ring of slots in static device memory; every launch must leave its
slot at zero, and a slot is reused only after its last launch has ended. These tests
check that results stay bit-identical when the ring wraps many times, when two streams
run the kernel at once, when 300 calls are queued on four streams without waiting, and
when the call is captured into a graph and replayed between eager calls.
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


def test_three_hundred_launches_on_four_streams():
    """300 calls queued on four streams with no synchronisation in between: more calls
    in flight than the ring has eager slots, on streams that do not order each other.
    Three different problems (each more work items than the grid has workgroups) take
    turns, so a slot shared by two running kernels would show as wrong output."""
    probs = [problem(20), problem(21, heads=16, frames=6, tokens=1560, w0=1560, d=128),
             problem(22, heads=12, frames=5, tokens=1000, w0=300, d=64)]
    refs = [radial.attn_fwd(*p) for p in probs]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream() for _ in range(4)]
    outs = []
    for i in range(300):
        p = i % 3
        out = torch.empty_like(refs[p])
        with torch.cuda.stream(streams[i % 4]):
            radial.attn_fwd(*probs[p], out=out)
        outs.append((p, out))
    torch.cuda.synchronize()
    for i, (p, out) in enumerate(outs):
        assert torch.equal(out, refs[p]), i


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


def random_table(nb, rng, singles):
    """A valid pair table: a random partition of the rows into pairs, `singles` rows alone."""
    perm = rng.permutation(nb)
    alone, rest = perm[:singles], perm[singles:]
    pairs = [sorted(rest[i:i + 2]) for i in range(0, len(rest) - 1, 2)]
    if len(rest) % 2:
        alone = list(alone) + [rest[-1]]
    rows = [(int(a), int(b)) for a, b in pairs] + [(int(a), -1) for a in alone]
    rows.sort()
    return torch.tensor(rows, dtype=torch.int32)


def test_pairing_does_not_change_results():
    """Each row's output depends only on its own key blocks, in ascending order: the
    greedy table, no table (adjacent pairs) and random tables give the same bits."""
    import numpy as np
    frames, tokens, w0 = 6, 1560, 1560
    g = torch.Generator(device="cuda").manual_seed(6)
    n = frames * tokens
    q, k, v = (torch.randn(1, 3, n, 128, generator=g, device="cuda").to(torch.bfloat16)
               for _ in range(3))
    host = radial.build_mask(frames, tokens, w0)
    nb = host.nb
    rng = np.random.default_rng(0)
    tables = [host.pairs, None, random_table(nb, rng, 0), random_table(nb, rng, 7)]
    outs = []
    for t in tables:
        m = radial.Mask(host.row_ptr, host.col_idx, frames, tokens, w0, t).to("cuda")
        lse = torch.empty(1, 3, n, dtype=torch.float32, device="cuda")
        outs.append((radial.attn_fwd(q, k, v, m, lse=lse), lse))
    torch.cuda.synchronize()
    for i, (o, lse) in enumerate(outs[1:], 1):
        assert torch.equal(o, outs[0][0]), i
        assert torch.equal(lse, outs[0][1]), i


def test_row_absent_from_table_is_not_written():
    """A table entry outside [0, nb) is an absent row: never read or written."""
    frames, tokens, w0 = 4, 1024, 512
    q, k, v, _ = problem(8, heads=2, frames=frames, tokens=tokens, w0=w0)
    host = radial.build_mask(frames, tokens, w0, pairs=False)
    nb = host.nb  # 32
    table = torch.tensor([[2 * p, 2 * p + 1] for p in range(nb // 2)], dtype=torch.int32)
    table[3, 1] = nb + 5   # row 7 is left out
    ref = radial.attn_fwd(q, k, v, host.to("cuda"))
    m = radial.Mask(host.row_ptr, host.col_idx, frames, tokens, w0, table).to("cuda")
    out = torch.full_like(q, 7.0)
    radial.attn_fwd(q, k, v, m, out=out)
    torch.cuda.synchronize()
    rows7 = slice(7 * 128, 8 * 128)
    assert torch.all(out[:, :, rows7] == 7.0)
    keep = torch.ones(out.shape[2], dtype=torch.bool)
    keep[rows7] = False
    assert torch.equal(out[:, :, keep], ref[:, :, keep])


def test_graph_capture_of_varlen_rule_and_backward():
    """The varlen forward, the on-the-fly mask and the backward pass, captured in one graph,
    replay bit-identically, with eager calls of the same entry points in between."""
    from block_sparse_attention_radial_amd.inputs import draw_packed_qkv
    masks = [radial.build_mask(f, 300, 40) for f in (5, 2, 7)]
    vm = radial.concat_masks(masks).to("cuda")
    total = sum(m.n for m in masks)
    pq, pk, pv = draw_packed_qkv(total, 2, 128, seed=41, device="cuda")
    q, k, v, mask = problem(6)
    rm = radial.rule_mask(mask.frames, mask.tokens_per_frame, mask.w0, pairs=True).to("cuda")
    g = torch.Generator(device="cuda").manual_seed(42)
    do = torch.randn(q.shape, generator=g, device="cuda").to(torch.bfloat16)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device="cuda")

    def work(outs):
        radial.attn_fwd_varlen(pq, pk, pv, vm, out=outs[0])
        radial.attn_fwd(q, k, v, rm, out=outs[1], lse=lse)
        grads = radial.attn_bwd(q, k, v, outs[1], do, lse, mask)
        for dst, src in zip(outs[2:], grads):
            dst.copy_(src)

    refs = [torch.empty_like(pq), torch.empty_like(q)] + [torch.empty_like(q) for _ in range(3)]
    work(refs)
    torch.cuda.synchronize()
    outs = [torch.empty_like(r) for r in refs]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        work(outs)  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        work(outs)
    eager = [torch.empty_like(r) for r in refs]
    for r in range(4):
        for o in outs:
            o.zero_()
        graph.replay()
        work(eager)
        torch.cuda.synchronize()
        for a, b, c in zip(outs, refs, eager):
            assert torch.equal(a, b), r
            assert torch.equal(c, b), r
