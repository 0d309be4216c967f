"""GPU parity of the backward pass (dq, dk, dv) against the oracle's attention_backward.

The GPU takes the forward's own bf16 output o and its lse; the oracle recomputes
everything in fp64 from the same bf16 q, k, v and do. The bar is relative to the size of
each gradient, since gradients, unlike the forward output, are not bounded by the inputs:

    max |got - ref| <= 2e-2 * max |ref|,   mean |got - ref| <= 5e-3 * mean |ref|.

Where it comes from: the outputs are rounded to bf16 (relative error up to 2^-9, about
2e-3, and about half that on average), and P and dS enter the matrix products as bf16,
adding errors of the same relative size that mostly cancel over the many terms of each
sum. On the shapes below the GPU measured at most 5.4e-3 (max) and 2.3e-3 (mean) of
those scales.
"""
import numpy as np
import pytest
import torch

import block_sparse_attention_radial_amd as radial
from block_sparse_attention_radial_amd.inputs import WORKLOADS, Workload, draw_qkv
from oracle import radial_oracle as ro

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
    ref = ro.attention_backward(f64(q), f64(k), f64(v), f64(do), mask.row_ptr.numpy(),
                                mask.col_idx.numpy(), D ** -0.5,
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
    ref = ro.attention_backward(f64(q), f64(k), f64(v), f64(do), mask.row_ptr.numpy(),
                                mask.col_idx.numpy(), wl.scale, query_blocks=qbs,
                                key_blocks=kbs)
    rows_q = np.concatenate([np.arange(b * 128, min(wl.n, b * 128 + 128)) for b in qbs])
    rows_k = np.concatenate([np.arange(b * 128, min(wl.n, b * 128 + 128)) for b in kbs])
    check(dq, ref[0], rows=rows_q)
    check(dk, ref[1], rows=rows_k)
    check(dv, ref[2], rows=rows_k)
