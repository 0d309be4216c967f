"""Element masking from a stored element table (radial_build_element_table,
radial_attn_fwd_element_table and radial_attn_bwd_element_table).

The table must hold exactly the rule's decisions, in the layout the kernel reads: every
stored bit of every active block is decoded here and compared with the oracle's n x n
element mask. The forward from the table must equal the forward that evaluates the rule
in the kernel, bit for bit (output and lse), and so inherits that path's oracle parity;
one small case is also checked against the oracle directly. The same holds for the
backward pass's gradients.
"""
import numpy as np
import pytest
import torch

import block_sparse_attention_radial_amd as radial
from block_sparse_attention_radial_amd.inputs import WORKLOADS, Workload, draw_qkv
from oracle import radial_oracle as ro
from oracle_masks import oracle_csr

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    radial.lib()


def decode(table, row_ptr, col_idx, n):
    """(query, key, bit) arrays for every stored decision of real tokens: entry j is CSR
    entry j, wave w holds queries 32w .. 32w + 31, lane l query 32w + l % 32, and bit
    16g + e key 32g + 8(e // 4) + 4(l // 32) + e % 4 of the block."""
    nnz = col_idx.size
    rows = np.repeat(np.arange(row_ptr.size - 1), np.diff(row_ptr))
    words = table.reshape(nnz, 4, 64).astype(np.uint64)
    w = np.arange(4)[None, :, None, None]
    lane = np.arange(64)[None, None, :, None]
    b = np.arange(64)[None, None, None, :]
    g, e = b // 16, b % 16
    q = rows[:, None, None, None] * 128 + 32 * w + lane % 32
    k = col_idx[:, None, None, None] * 128 + 32 * g + 8 * (e // 4) + 4 * (lane // 32) + e % 4
    bits = (words[..., None] >> b.astype(np.uint64)) & np.uint64(1)
    q, k, bits = np.broadcast_arrays(q, k, bits)
    real = (q < n) & (k < n)
    return q[real], k[real], bits[real].astype(bool)


TABLE_CASES = [
    # name, F, S, W0, grid width (None: 1-D distance)
    ("eight-frames", 8, 512, 256, None),
    ("narrow", 6, 300, 40, None),
    ("ragged", 5, 1000, 334, None),
    ("frame-straddle", 7, 130, 60, None),
    ("grid-rows-of-20", 5, 320, 9, 20),
    ("grid-rows-of-8", 4, 256, 5, 8),
]


@pytest.mark.parametrize("name,F,S,w0,gw", TABLE_CASES, ids=[c[0] for c in TABLE_CASES])
def test_table_holds_the_oracle_element_mask(name, F, S, w0, gw):
    mask = radial.build_mask(F, S, w0, grid_w=gw)
    table = radial.build_element_table(mask.to("cuda"))
    torch.cuda.synchronize()
    rp, ci = mask.row_ptr.numpy(), mask.col_idx.numpy()
    assert table.shape == (ci.size, 256)
    q, k, bits = decode(table.cpu().numpy().view(np.uint64), rp, ci, F * S)
    ref = ro.element_mask(F, S, w0, grid_w=gw)
    np.testing.assert_array_equal(bits, ref[q, k])
    # Every real (query, key) pair of every active block is covered exactly once.
    arp, aci = oracle_csr(F, S, w0, gw)
    n = F * S
    cover = np.zeros((n, n), dtype=np.int32)
    np.add.at(cover, (q, k), 1)
    active = np.zeros((n, n), dtype=bool)
    for r in range(arp.size - 1):
        for c in aci[arp[r]:arp[r + 1]]:
            active[r * 128:(r + 1) * 128, c * 128:(c + 1) * 128] = True
    np.testing.assert_array_equal(cover, active.astype(np.int32))


def fwd_both(wl, gw=None, pairs=True, seed=4, heads=None, device_draw=False):
    """The element forward evaluating the rule in the kernel and from the table."""
    if device_draw:
        q, k, v = draw_qkv(wl, seed=seed, device="cuda")
    else:
        q, k, v = (x.cuda() for x in draw_qkv(wl, seed=seed))
    if heads is not None:
        q, k, v = (x[:, heads].contiguous() for x in (q, k, v))
    B, H, n, _ = q.shape
    mask = radial.build_mask(wl.frames, wl.tokens_per_frame, wl.w0, pairs=pairs,
                             grid_w=gw).to("cuda")
    outs = []
    for use_table in (False, True):
        m = radial.Mask(**{**mask.__dict__, "element_table": None})
        if use_table:
            m.with_element_table()
        lse = torch.full((B, H, n), float("nan"), dtype=torch.float32, device="cuda")
        o = torch.full_like(q, float("nan"))
        radial.attn_fwd(q, k, v, m, out=o, lse=lse, element=True)
        outs.append((o, lse))
    torch.cuda.synchronize()
    return outs, (q, k, v), mask


SMALL = [
    # name, B, H, D, F, S, W0, grid width
    ("small", 1, 8, 64, 8, 1024, 512, None),
    ("narrow-d128", 2, 2, 128, 6, 300, 40, None),
    ("narrow-d64", 1, 3, 64, 9, 200, 9, None),
    ("ragged-d128", 1, 2, 128, 5, 1000, 334, None),
    ("frame-straddle", 1, 2, 128, 7, 130, 60, None),
    ("one-frame", 1, 2, 128, 1, 2000, 100, None),
    ("grid-rows-of-20", 1, 2, 128, 5, 320, 9, 20),
    ("grid-rows-of-50", 2, 2, 64, 4, 1500, 31, 50),
]


@pytest.mark.parametrize("pairs", [True, False], ids=["pair-table", "rows-2p"])
@pytest.mark.parametrize("name,B,H,D,F,S,w0,gw", SMALL, ids=[c[0] for c in SMALL])
def test_table_forward_equals_rule_forward(name, B, H, D, F, S, w0, gw, pairs):
    wl = Workload(name, B, H, D, F, S, w0, 1.0)
    ((o_rule, l_rule), (o_tab, l_tab)), _, _ = fwd_both(wl, gw, pairs)
    assert torch.isfinite(o_tab.float()).all() and torch.isfinite(l_tab).all()
    assert torch.equal(o_tab.view(torch.int16), o_rule.view(torch.int16))
    assert torch.equal(l_tab.view(torch.int32), l_rule.view(torch.int32))


def test_table_forward_against_oracle():
    wl = Workload("narrow", 1, 2, 128, 6, 300, 40, 1.0)
    ((_, _), (o, lse)), (q, k, v), mask = fwd_both(wl)
    rp, ci = oracle_csr(6, 300, 40)
    f64 = lambda x: x.detach().to("cpu", torch.float64).numpy()  # noqa: E731
    ref, ref_lse = ro.attention(f64(q), f64(k), f64(v), rp, ci, wl.scale, element=(300, 40))
    err = np.abs(f64(o) - ref)
    assert err.max() <= 2e-2 and err.mean() <= 2e-3, (err.max(), err.mean())
    assert np.abs(f64(lse) - ref_lse).max() < 1e-3


@pytest.mark.parametrize("key", ["wan", "wan-grid", "hunyuan", "long4x"])
def test_table_forward_equals_rule_forward_full_size(key):
    """The full-size workloads (Wan 1-D and grid distance, HunyuanVideo, 4x long), every
    head: many items per workgroup, both groups of every pair, every table entry in use
    (up to 357,580 entries, 732 MB)."""
    wl = WORKLOADS[key]
    ((o_rule, l_rule), (o_tab, l_tab)), _, _ = fwd_both(wl, gw=wl.grid_w, device_draw=True)
    assert torch.isfinite(l_tab).all()
    assert torch.equal(o_tab.view(torch.int16), o_rule.view(torch.int16))
    assert torch.equal(l_tab.view(torch.int32), l_rule.view(torch.int32))


def test_autograd_with_a_table_mask_equals_the_rule_mask():
    """attention() with a table-carrying mask: the forward reads the table, the backward
    takes the same decisions from the rule, so values and gradients are unchanged."""
    wl = Workload("narrow", 1, 2, 128, 6, 300, 40, 1.0)
    q, k, v = draw_qkv(wl, seed=6)
    do = torch.randn(q.shape, generator=torch.Generator().manual_seed(7)).to(torch.bfloat16)
    mask = radial.build_mask(6, 300, 40).to("cuda")
    results = []
    for use_table in (False, True):
        m = radial.Mask(**{**mask.__dict__, "element_table": None})
        if use_table:
            m.with_element_table()
        qd, kd, vd = (x.cuda().requires_grad_() for x in (q, k, v))
        o = radial.attention(qd, kd, vd, m, element=True)
        o.backward(do.cuda())
        results.append([o.detach(), qd.grad, kd.grad, vd.grad])
    torch.cuda.synchronize()
    for a, b in zip(*results):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_python_wrapper_checks_the_table():
    wl = Workload("narrow", 1, 1, 128, 6, 300, 40, 1.0)
    q, k, v = (x.cuda() for x in draw_qkv(wl, seed=8))
    mask = radial.build_mask(6, 300, 40).to("cuda").with_element_table()
    bad = radial.Mask(**{**mask.__dict__, "element_table": mask.element_table[:-1]})
    with pytest.raises(ValueError):
        radial.attn_fwd(q, k, v, bad, element=True)
    with pytest.raises(ValueError):
        radial.build_element_table(radial.build_mask(6, 300, 40))  # a CPU mask
    with pytest.raises(ValueError):
        radial.build_element_table(radial.build_mask(6, 100, 40).to("cuda"))  # frame < 128


def bwd_both(wl, gw=None, seed=9, mask=None):
    """Element-masked gradients evaluating the rule in the kernels and from the table,
    on the same forward output and lse."""
    q, k, v = (x.cuda() for x in draw_qkv(wl, seed=seed))
    g = torch.Generator().manual_seed(seed + 1)
    do = torch.randn(q.shape, generator=g).to(torch.bfloat16).cuda()
    if mask is None:
        mask = radial.build_mask(wl.frames, wl.tokens_per_frame, wl.w0, grid_w=gw)
    mask = mask.to("cuda")
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device="cuda")
    o = radial.attn_fwd(q, k, v, mask, lse=lse, element=True)
    grads = []
    for use_table in (False, True):
        m = radial.Mask(**{**mask.__dict__, "element_table": None})
        if use_table:
            m.with_element_table()
        grads.append(radial.attn_bwd(q, k, v, o, do, lse, m, element=True))
    torch.cuda.synchronize()
    return grads


@pytest.mark.parametrize("name,B,H,D,F,S,w0,gw", SMALL, ids=[c[0] for c in SMALL])
def test_table_backward_equals_rule_backward(name, B, H, D, F, S, w0, gw):
    wl = Workload(name, B, H, D, F, S, w0, 1.0)
    rule, table = bwd_both(wl, gw)
    for a, b in zip(rule, table):
        assert torch.isfinite(b.float()).all()
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))


@pytest.mark.parametrize("key", ["wan", "wan-grid"])
def test_table_backward_equals_rule_backward_full_size(key):
    wl = WORKLOADS[key]
    wl = Workload(wl.name, 1, 2, wl.head_dim, wl.frames, wl.tokens_per_frame, wl.w0, 1.0,
                  grid_w=wl.grid_w)  # two of the 40 heads: every block of the mask
    rule, table = bwd_both(wl, wl.grid_w)
    for a, b in zip(rule, table):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_table_backward_of_a_mask_that_is_not_symmetric():
    """A CSR whose transpose differs (row 0 sees every block, the others only the
    diagonal): the forward reads the table, the backward falls back to the rule (dK/dV
    walks columns), and everything equals the rule path."""
    nb, F, S = 6, 4, 192
    rows = [list(range(nb))] + [[r] for r in range(1, nb)]
    row_ptr = torch.tensor(np.cumsum([0] + [len(r) for r in rows]), dtype=torch.int32)
    col_idx = torch.tensor([c for r in rows for c in r], dtype=torch.int32)
    mask = radial.Mask(row_ptr, col_idx, F, S, 50)
    assert not mask.symmetric()
    wl = Workload("asym", 1, 2, 128, F, S, 50, 1.0)
    rule, table = bwd_both(wl, mask=mask)
    for a, b in zip(rule, table):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_graph_capture_of_the_table_paths():
    """The table forward and backward captured in one graph (the table built outside it)
    replay bit-identically, with eager rule-path calls in between."""
    wl = Workload("narrow", 1, 2, 128, 6, 300, 40, 1.0)
    q, k, v = (x.cuda() for x in draw_qkv(wl, seed=11))
    g = torch.Generator(device="cuda").manual_seed(12)
    do = torch.randn(q.shape, generator=g, device="cuda").to(torch.bfloat16)
    mask = radial.build_mask(6, 300, 40).to("cuda").transposed()
    tab = radial.Mask(**{**mask.__dict__, "element_table": None}).with_element_table()
    assert tab.symmetric()
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device="cuda")

    def work(outs, m):
        radial.attn_fwd(q, k, v, m, out=outs[0], lse=lse, element=True)
        for dst, src in zip(outs[1:], radial.attn_bwd(q, k, v, outs[0], do, lse, m,
                                                       element=True)):
            dst.copy_(src)

    refs = [torch.empty_like(q) for _ in range(4)]
    work(refs, mask)  # the rule path: the reference
    torch.cuda.synchronize()
    outs = [torch.empty_like(q) for _ in range(4)]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        work(outs, tab)  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        work(outs, tab)
    scratch = [torch.empty_like(q) for _ in range(4)]
    for r in range(4):
        for o in outs:
            o.zero_()
        graph.replay()
        work(scratch, mask)
        torch.cuda.synchronize()
        for a, b in zip(outs, refs):
            assert torch.equal(a.view(torch.int16), b.view(torch.int16)), r


VARLEN = [
    # frames per sample, S, W0, grid width, heads, head_dim
    ([5, 2, 7], 300, 40, None, 2, 128),
    ([3, 6, 1], 320, 9, 20, 2, 64),
    ([21, 16, 11, 5], 1560, 1560, None, 2, 128),  # the Wan-shaped batch, two heads
]


@pytest.mark.parametrize("frames,S,w0,gw,H,D", VARLEN, ids=["narrow", "grid", "wan-batch"])
def test_varlen_table_equals_varlen_rule(frames, S, w0, gw, H, D):
    """A packed batch: forward (output, lse) and gradients from the concatenated tables
    equal the varlen path that evaluates the rule, bit for bit."""
    from block_sparse_attention_radial_amd.inputs import draw_packed_qkv
    masks = [radial.build_mask(f, S, w0, grid_w=gw) for f in frames]
    vm = radial.concat_masks(masks).to("cuda")
    total = sum(m.n for m in masks)
    q, k, v = draw_packed_qkv(total, H, D, seed=21, device="cuda")
    g = torch.Generator(device="cuda").manual_seed(22)
    do = torch.randn(q.shape, generator=g, device="cuda").to(torch.bfloat16)
    results = []
    for use_table in (False, True):
        m = radial.VarlenMask(**{**vm.__dict__, "element_table": None})
        if use_table:
            m.with_element_table()
            assert m.element_table.shape == (vm.col_idx.numel(), 256)
            assert m.symmetric()
        lse = torch.empty(H, total, dtype=torch.float32, device="cuda")
        o = radial.attn_fwd_varlen(q, k, v, m, lse=lse, element=True)
        grads = radial.attn_bwd_varlen(q, k, v, o, do, lse, m, element=True)
        results.append([o, lse.view(torch.int16)] + list(grads))
    torch.cuda.synchronize()
    for i, (a, b) in enumerate(zip(*results)):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16)), i


def test_table_forward_with_random_pair_tables():
    """Random pair tables, some rows alone (the other group of such a workgroup has no
    row): each group counts its own row's entries, so every table gives the bits of the
    rule path."""
    def random_table(nb, rng, singles):
        perm = rng.permutation(nb)
        alone, rest = list(perm[:singles]), perm[singles:]
        rows = [tuple(sorted(int(x) for x in rest[i:i + 2])) for i in range(0, len(rest) - 1, 2)]
        if len(rest) % 2:
            alone.append(rest[-1])
        rows = sorted(rows + [(int(a), -1) for a in alone])
        return torch.tensor(rows, dtype=torch.int32)

    wl = Workload("narrow", 1, 3, 128, 6, 300, 40, 1.0)
    q, k, v = (x.cuda() for x in draw_qkv(wl, seed=31))
    host = radial.build_mask(6, 300, 40, pairs=False)
    ref = radial.attn_fwd(q, k, v, host.to("cuda"), element=True)
    rng = np.random.default_rng(5)
    for singles in (0, 3, host.nb):
        t = random_table(host.nb, rng, singles)
        m = radial.Mask(host.row_ptr, host.col_idx, 6, 300, 40, t).to("cuda").with_element_table()
        o = radial.attn_fwd(q, k, v, m, element=True)
        torch.cuda.synchronize()
        assert torch.equal(o.view(torch.int16), ref.view(torch.int16)), singles
