"""GPU parity of the backward pass (dq, dk, dv) against the oracle's attention_backward.

The GPU takes the forward's own bf16 output o and its lse; the oracle recomputes
everything in fp64 from the same bf16 q, k, v and do. The bar is relative to the size of
each gradient, since gradients, unlike the forward output, are not bounded by the inputs:

    max |got - ref| <= 2e-2 * max |ref|,   mean |got - ref| <= 5e-3 * mean |ref|.

Where it comes from: the outputs are rounded to bf16 (relative error up to 2^-9, about
2e-3, and about half that on average), and P and dS enter the matrix products as bf16,
adding errors of the same relative size that mostly cancel over the many terms of each
sum (dS is formed from the bf16-rounded P that also enters dV's product). On the small
shapes below the GPU measured at most 7.2e-3 (max, dk with element masking) and 2.8e-3
(mean, dk) of those scales.
"""
import numpy as np
import pytest
import torch

import block_sparse_attention_radial_amd as radial
from block_sparse_attention_radial_amd.inputs import WORKLOADS, Workload, draw_qkv
from oracle import radial_oracle as ro
from oracle_masks import oracle_csr

pytestmark = pytest.mark.gpu

MAX_REL, MEAN_REL = 2e-2, 5e-3


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    radial.lib()


def f64(x):
    return x.detach().to("cpu", torch.float64).numpy()


def check(got, ref, rows=None):
    got = f64(got)
    if rows is not None:
        got, ref = got[..., rows, :], ref[..., rows, :]
    assert np.isfinite(got).all()
    err = np.abs(got - ref)
    assert err.max() <= MAX_REL * np.abs(ref).max(), (err.max(), np.abs(ref).max())
    assert err.mean() <= MEAN_REL * np.abs(ref).mean(), (err.mean(), np.abs(ref).mean())


def run(wl, element=False, seed=3, mask=None):
    q, k, v = draw_qkv(wl, seed=seed)
    g = torch.Generator().manual_seed(seed + 100)
    do = torch.randn(wl.batch, wl.heads, wl.n, wl.head_dim, generator=g).to(torch.bfloat16)
    mask = mask or radial.build_mask(wl.frames, wl.tokens_per_frame, wl.w0)
    md = mask.to("cuda")
    qc, kc, vc, dc = (x.cuda() for x in (q, k, v, do))
    lse = torch.empty(wl.batch, wl.heads, wl.n, dtype=torch.float32, device="cuda")
    o = radial.attn_fwd(qc, kc, vc, md, lse=lse, element=element)
    grads = radial.attn_bwd(qc, kc, vc, o, dc, lse, md, element=element)
    torch.cuda.synchronize()
    return (q, k, v, do), mask, grads


SMALL = [
    # name, B, H, D, F, S, W0, element
    ("tiny", 1, 1, 64, 4, 256, 256, False),
    ("sparse-d128", 1, 2, 128, 6, 1000, 100, False),
    ("sparse-d64", 2, 2, 64, 6, 1000, 100, False),
    ("ragged", 1, 2, 128, 5, 1000, 334, False),
    ("one-block", 1, 1, 128, 1, 100, 7, False),
    ("element-narrow", 1, 2, 128, 6, 300, 40, True),
    ("element-d64", 1, 2, 64, 9, 200, 9, True),
    ("wan-frames", 1, 1, 128, 8, 1560, 1560, False),
]


@pytest.mark.parametrize("name,B,H,D,F,S,w0,element", SMALL, ids=[c[0] for c in SMALL])
def test_backward_parity_small(name, B, H, D, F, S, w0, element):
    wl = Workload(name, B, H, D, F, S, w0, 1.0)
    (q, k, v, do), mask, grads = run(wl, element)
    ref = ro.attention_backward(f64(q), f64(k), f64(v), f64(do), *oracle_csr(F, S, w0),
                                D ** -0.5,
                                element=(S, w0) if element else None)
    for got, r in zip(grads, ref):
        check(got, r)


def test_backward_non_symmetric_mask_uses_the_transpose():
    """A random, non-symmetric block mask: dk and dv need its transpose."""
    rng = np.random.default_rng(11)
    n, D = 128 * 9 + 40, 128
    nb = (n + 127) // 128
    rows = [np.flatnonzero((rng.random(nb) < 0.35) | (np.arange(nb) == r)).astype(np.int32)
            for r in range(nb)]
    rp = np.zeros(nb + 1, np.int32)
    rp[1:] = np.cumsum([len(r) for r in rows])
    mask = radial.Mask(torch.from_numpy(rp), torch.from_numpy(np.concatenate(rows)), 1, n, 1)
    wl = Workload("random", 1, 2, D, 1, n, 1, 1.0)
    (q, k, v, do), mask, grads = run(wl, mask=mask)
    ref = ro.attention_backward(f64(q), f64(k), f64(v), f64(do), rp, np.concatenate(rows),
                                D ** -0.5)
    for got, r in zip(grads, ref):
        check(got, r)


def test_autograd_matches_attn_bwd():
    wl = Workload("autograd", 1, 2, 128, 4, 1000, 200, 1.0)
    q, k, v = (x.cuda().requires_grad_() for x in draw_qkv(wl, seed=5))
    mask = radial.build_mask(4, 1000, 200).to("cuda")
    do = torch.randn_like(q)
    o = radial.attention(q, k, v, mask)
    o.backward(do)
    lse = torch.empty(1, 2, wl.n, dtype=torch.float32, device="cuda")
    o2 = radial.attn_fwd(q.detach(), k.detach(), v.detach(), mask, lse=lse)
    ref = radial.attn_bwd(q.detach(), k.detach(), v.detach(), o2, do, lse, mask)
    torch.cuda.synchronize()
    assert torch.equal(o, o2)
    for a, b in zip((q.grad, k.grad, v.grad), ref):
        assert torch.equal(a, b)


def test_autograd_of_a_sum():
    """o.sum().backward(): the output gradient arrives as an expanded tensor with zero
    strides; it is copied into q's strides before the backward kernels read it."""
    wl = Workload("sum", 1, 2, 128, 4, 1000, 200, 1.0)
    q, k, v = draw_qkv(wl, seed=6)
    mask = radial.build_mask(4, 1000, 200)
    qc, kc, vc = (x.cuda().requires_grad_() for x in (q, k, v))
    radial.attention(qc, kc, vc, mask.to("cuda")).sum().backward()
    torch.cuda.synchronize()
    do = torch.ones(q.shape, dtype=torch.bfloat16)
    ref = ro.attention_backward(f64(q), f64(k), f64(v), f64(do), *oracle_csr(4, 1000, 200),
                                wl.scale)
    for got, r in zip((qc.grad, kc.grad, vc.grad), ref):
        check(got, r)


def test_autograd_with_bnhd_views():
    """q, k, v stored [B, n, H, D] and viewed as [B, H, n, D]; the output gradient comes
    contiguous in [B, H, n, D] (other strides than q's) and is copied into q's strides."""
    wl = Workload("bnhd", 2, 3, 128, 4, 500, 150, 1.0)
    q, k, v = draw_qkv(wl, seed=8)
    g = torch.Generator().manual_seed(9)
    do = torch.randn(q.shape, generator=g).to(torch.bfloat16)
    mask = radial.build_mask(4, 500, 150)
    views = [x.transpose(1, 2).contiguous().cuda().transpose(1, 2).requires_grad_()
             for x in (q, k, v)]
    assert views[0].stride() != do.stride()
    o = radial.attention(*views, mask.to("cuda"))
    o.backward(do.cuda())
    torch.cuda.synchronize()
    ref = ro.attention_backward(f64(q), f64(k), f64(v), f64(do), *oracle_csr(4, 500, 150),
                                wl.scale)
    for got, r in zip((x.grad for x in views), ref):
        check(got, r)


def test_backward_scale_zero_ragged():
    """scale = 0 on a ragged shape: P is uniform over each row's real keys, so dq and dk
    are exactly zero and dv is the mean of dO over the rows that reach each key; padded
    keys must not turn into NaN."""
    wl = Workload("s0", 1, 2, 128, 5, 1000, 100, 1.0)
    q, k, v = draw_qkv(wl, seed=10)
    g = torch.Generator().manual_seed(11)
    do = torch.randn(q.shape, generator=g).to(torch.bfloat16)
    mask = radial.build_mask(5, 1000, 100)
    md = mask.to("cuda")
    qc, kc, vc, dc = (x.cuda() for x in (q, k, v, do))
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device="cuda")
    o = radial.attn_fwd(qc, kc, vc, md, scale=0.0, lse=lse)
    dq, dk, dv = radial.attn_bwd(qc, kc, vc, o, dc, lse, md, scale=0.0)
    torch.cuda.synchronize()
    ref = ro.attention_backward(f64(q), f64(k), f64(v), f64(do), *oracle_csr(5, 1000, 100),
                                0.0)
    assert not np.abs(ref[0]).any() and not np.abs(ref[1]).any()
    assert bool((dq == 0).all()) and bool((dk == 0).all())
    check(dv, ref[2])


def test_backward_full_size_sampled_wan():
    """Wan shape (two heads): dq on sampled query blocks, dk and dv on sampled key
    blocks (the oracle processes every query block that reaches them)."""
    wl = WORKLOADS["wan"]
    heads = range(2)
    q, k, v = draw_qkv(wl, seed=0, device="cuda", heads=heads)
    g = torch.Generator(device="cuda").manual_seed(7)
    do = torch.randn(q.shape, generator=g, device="cuda").to(torch.bfloat16)
    mask = radial.build_mask(wl.frames, wl.tokens_per_frame, wl.w0)
    md = mask.to("cuda")
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device="cuda")
    o = radial.attn_fwd(q, k, v, md, lse=lse)
    dq, dk, dv = radial.attn_bwd(q, k, v, o, do, lse, md)
    torch.cuda.synchronize()
    qbs, kbs = [0, 131, wl.nb - 1], [3, wl.nb - 1]
    ref = ro.attention_backward(f64(q), f64(k), f64(v), f64(do),
                                *oracle_csr(wl.frames, wl.tokens_per_frame, wl.w0),
                                wl.scale, query_blocks=qbs,
                                key_blocks=kbs)
    rows_q = np.concatenate([np.arange(b * 128, min(wl.n, b * 128 + 128)) for b in qbs])
    rows_k = np.concatenate([np.arange(b * 128, min(wl.n, b * 128 + 128)) for b in kbs])
    check(dq, ref[0], rows=rows_q)
    check(dk, ref[1], rows=rows_k)
    check(dv, ref[2], rows=rows_k)


def _mask_from_rows(rows, n):
    rp = np.zeros(len(rows) + 1, np.int32)
    rp[1:] = np.cumsum([len(r) for r in rows])
    ci = np.concatenate([np.asarray(r, np.int32) for r in rows])
    return rp, ci, radial.Mask(torch.from_numpy(rp), torch.from_numpy(ci), 1, n, 1)


def test_backward_empty_column_and_ragged_tail():
    """Key block 4 is listed by no row (its dk/dv walk has no query tiles and must come
    out exactly zero); rows of one to four blocks; n ends 50 tokens into block 5, so the
    last query tile's second half holds no rows."""
    n, D = 128 * 6 - 50, 128
    rows = [[0], [0, 1], [1, 2], [0, 3], [0, 1, 2, 3], [5]]
    rp, ci, mask = _mask_from_rows(rows, n)
    wl = Workload("empty-column", 1, 2, D, 1, n, 1, 1.0)
    (q, k, v, do), _, grads = run(wl, mask=mask)
    ref = ro.attention_backward(f64(q), f64(k), f64(v), f64(do), rp, ci, D ** -0.5)
    for got, r in zip(grads, ref):
        check(got, r)
    keys4 = slice(4 * 128, 5 * 128)
    assert bool((grads[1][..., keys4, :] == 0).all()) and bool((grads[2][..., keys4, :] == 0).all())


def test_backward_skips_out_of_range_columns():
    """Column indices outside [0, nb) are skipped (as in the forward): the gradients equal
    the oracle's on the CSR without them, and the library's own on that CSR bit for bit."""
    n, D = 128 * 4 + 17, 64
    nb = 5
    clean = [[0, 2], [1], [0, 1, 2], [3, 4], [2, 4]]
    dirty = [[-1, 0, 2], [1, nb], [0, 1, 2, 7], [3, 4], [-5, 2, 4, nb + 3]]
    rp, ci, mask_clean = _mask_from_rows(clean, n)
    _, _, mask_dirty = _mask_from_rows(dirty, n)
    wl = Workload("dirty", 1, 2, D, 1, n, 1, 1.0)
    (q, k, v, do), _, grads = run(wl, mask=mask_dirty)
    _, _, grads_clean = run(wl, mask=mask_clean)
    ref = ro.attention_backward(f64(q), f64(k), f64(v), f64(do), rp, ci, D ** -0.5)
    for got, r in zip(grads, ref):
        check(got, r)
    for a, b in zip(grads, grads_clean):
        assert torch.equal(a, b)


@pytest.mark.parametrize("head_dim", [128, 64])
def test_backward_full_size_one_head_wan(head_dim):
    """Every dq, dk and dv row of one Wan-shaped head (n = 32760, 256 blocks, every
    column of the mask walked), against the oracle over the whole head; at D = 128 (the
    Wan head) and D = 64 (the kernels' other instance, same mask)."""
    w = WORKLOADS["wan"]
    wl = Workload(w.name, 1, w.heads, head_dim, w.frames, w.tokens_per_frame, w.w0, w.sigma)
    q, k, v = draw_qkv(wl, seed=0, device="cuda", heads=range(1))
    g = torch.Generator(device="cuda").manual_seed(12)
    do = torch.randn(q.shape, generator=g, device="cuda").to(torch.bfloat16)
    md = radial.build_mask(wl.frames, wl.tokens_per_frame, wl.w0).to("cuda")
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device="cuda")
    o = radial.attn_fwd(q, k, v, md, lse=lse)
    grads = radial.attn_bwd(q, k, v, o, do, lse, md)
    torch.cuda.synchronize()
    ref = ro.attention_backward(f64(q), f64(k), f64(v), f64(do),
                                *oracle_csr(wl.frames, wl.tokens_per_frame, wl.w0), wl.scale)
    for got, r in zip(grads, ref):
        check(got, r)


@pytest.mark.parametrize("wlname", ["wan", "wan-grid"])
def test_backward_full_size_sampled_element(wlname):
    """Element masking at full size (the 1-D rule at Wan, the grid rule at the Wan grid),
    one head: dq on sampled query blocks, dk and dv on sampled key blocks (the first,
    one inside, the ragged last), against the oracle's element option."""
    wl = WORKLOADS[wlname]
    q, k, v = draw_qkv(wl, seed=0, device="cuda", heads=range(1))
    g = torch.Generator(device="cuda").manual_seed(13)
    do = torch.randn(q.shape, generator=g, device="cuda").to(torch.bfloat16)
    md = radial.build_mask(wl.frames, wl.tokens_per_frame, wl.w0, grid_w=wl.grid_w).to("cuda")
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device="cuda")
    o = radial.attn_fwd(q, k, v, md, lse=lse, element=True)
    dq, dk, dv = radial.attn_bwd(q, k, v, o, do, lse, md, element=True)
    torch.cuda.synchronize()
    qbs, kbs = [0, 97, wl.nb - 1], [5, 200, wl.nb - 1]
    element = ((wl.tokens_per_frame, wl.w0) if wl.grid_w is None
               else (wl.tokens_per_frame, wl.w0, wl.grid_w))
    ref = ro.attention_backward(f64(q), f64(k), f64(v), f64(do),
                                *oracle_csr(wl.frames, wl.tokens_per_frame, wl.w0, wl.grid_w),
                                wl.scale, element=element, query_blocks=qbs, key_blocks=kbs)
    rows_q = np.concatenate([np.arange(b * 128, min(wl.n, b * 128 + 128)) for b in qbs])
    rows_k = np.concatenate([np.arange(b * 128, min(wl.n, b * 128 + 128)) for b in kbs])
    check(dq, ref[0], rows=rows_q)
    check(dk, ref[1], rows=rows_k)
    check(dv, ref[2], rows=rows_k)


@pytest.mark.parametrize("wlname", ["hunyuan", "long4x"])
def test_backward_full_size_sampled_large(wlname):
    """The two large workloads at full size, one head: dq on sampled query blocks (the
    first, a middle one, the ragged last) and dk, dv on the ragged last key block, whose
    column reaches hundreds of query blocks (the oracle recomputes each of their rows in
    full, which bounds what can be sampled)."""
    wl = WORKLOADS[wlname]
    q, k, v = draw_qkv(wl, seed=0, device="cuda", heads=range(1))
    g = torch.Generator(device="cuda").manual_seed(14)
    do = torch.randn(q.shape, generator=g, device="cuda").to(torch.bfloat16)
    md = radial.build_mask(wl.frames, wl.tokens_per_frame, wl.w0).to("cuda")
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device="cuda")
    o = radial.attn_fwd(q, k, v, md, lse=lse)
    dq, dk, dv = radial.attn_bwd(q, k, v, o, do, lse, md)
    torch.cuda.synchronize()
    qbs, kbs = [0, wl.nb // 2, wl.nb - 1], [wl.nb - 1]
    ref = ro.attention_backward(f64(q), f64(k), f64(v), f64(do),
                                *oracle_csr(wl.frames, wl.tokens_per_frame, wl.w0),
                                wl.scale, query_blocks=qbs, key_blocks=kbs)
    rows_q = np.concatenate([np.arange(b * 128, min(wl.n, b * 128 + 128)) for b in qbs])
    rows_k = np.arange((wl.nb - 1) * 128, wl.n)
    check(dq, ref[0], rows=rows_q)
    check(dk, ref[1], rows=rows_k)
    check(dv, ref[2], rows=rows_k)
