"""GPU parity of element masking: the radial rule applied to single entries inside the
active blocks, against the oracle's element option, on the same seeded inputs.

Bar as for block semantics: max-abs 2e-2, mean-abs 2e-3 over every checked element, lse
within 1e-3. Small shapes are compared in full; the full-size workloads on sampled query
blocks of three heads. Narrow windows make whole tiles masked for some rows, including
a row's first tiles, which exercises the kernel's late setting of the reference max.
"""
import numpy as np
import pytest
import torch

import block_sparse_attention_radial_amd as radial
from block_sparse_attention_radial_amd.inputs import WORKLOADS, Workload, draw_qkv
from oracle import radial_oracle as ro
from oracle_masks import oracle_csr

pytestmark = pytest.mark.gpu

MAX_ABS, MEAN_ABS = 2e-2, 2e-3


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    radial.lib()


def f64(x):
    return x.detach().to("cpu", torch.float64).numpy()


def oracle_element(q, k, v, mask, scale, query_blocks=None):
    rp, ci = oracle_csr(mask.frames, mask.tokens_per_frame, mask.w0)
    return ro.attention(f64(q), f64(k), f64(v), rp, ci, scale, query_blocks=query_blocks,
                        element=(mask.tokens_per_frame, mask.w0))


def check(o_gpu, o_ref, rows=None):
    got = f64(o_gpu)
    if rows is not None:
        got, o_ref = got[..., rows, :], o_ref[..., rows, :]
    err = np.abs(got - o_ref)
    assert np.isfinite(got).all()
    assert err.max() <= MAX_ABS and err.mean() <= MEAN_ABS, (err.max(), err.mean())


SMALL = [
    # name, B, H, D, F, S, W0
    ("tiny", 1, 1, 64, 4, 256, 256),
    ("small", 1, 8, 64, 8, 1024, 512),
    ("narrow-d128", 2, 2, 128, 6, 300, 40),     # many partial and fully masked tiles
    ("narrow-d64", 1, 3, 64, 9, 200, 9),
    ("ragged-d128", 1, 2, 128, 5, 1000, 334),  # n = 5000: ragged last block
    ("frame-straddle", 1, 2, 128, 7, 130, 60),  # almost every tile spans two frames
    ("one-frame", 1, 2, 128, 1, 2000, 100),     # a sliding window |i - j| < 100
]


@pytest.mark.parametrize("name,B,H,D,F,S,w0", SMALL, ids=[c[0] for c in SMALL])
def test_element_parity_small(name, B, H, D, F, S, w0):
    wl = Workload(name, B, H, D, F, S, w0, 1.0)
    q, k, v = draw_qkv(wl, seed=1)
    mask = radial.build_mask(F, S, w0)
    lse = torch.empty(B, H, wl.n, dtype=torch.float32, device="cuda")
    o = radial.attn_fwd(q.cuda(), k.cuda(), v.cuda(), mask.to("cuda"), lse=lse, element=True)
    torch.cuda.synchronize()
    ref, ref_lse = oracle_element(q, k, v, mask, wl.scale)
    check(o, ref)
    assert np.abs(f64(lse) - ref_lse).max() < 1e-3


def test_element_differs_from_block_semantics():
    """A narrow window: element masking changes the output (the same inputs under block
    semantics are a different softmax)."""
    wl = Workload("narrow", 1, 1, 128, 6, 300, 40, 1.0)
    q, k, v = (x.cuda() for x in draw_qkv(wl, seed=2))
    mask = radial.build_mask(6, 300, 40).to("cuda")
    o_el = radial.attn_fwd(q, k, v, mask, element=True)
    o_bl = radial.attn_fwd(q, k, v, mask)
    torch.cuda.synchronize()
    assert (o_el.float() - o_bl.float()).abs().max().item() > 0.05


def test_element_scale_zero_is_mean_over_allowed_keys():
    """scale = 0: every allowed key weighs the same, so the output is the mean of V over
    the allowed keys; this pins the kernel's key set exactly."""
    F, S, w0, D = 5, 256, 30, 64
    n = F * S
    g = torch.Generator().manual_seed(3)
    v = torch.randn(1, 1, n, D, generator=g).to(torch.bfloat16)
    q = torch.zeros_like(v)
    mask = radial.build_mask(F, S, w0)
    o = radial.attn_fwd(q.cuda(), q.cuda(), v.cuda(), mask.to("cuda"), scale=0.0, element=True)
    torch.cuda.synchronize()
    t = np.arange(n)
    vv = f64(v)[0, 0]
    got = f64(o)[0, 0]
    for i in range(0, n, 17):
        keys = ro.allowed(i // S, i % S, t // S, t % S, w0)
        assert np.abs(got[i] - vv[keys].mean(axis=0)).max() < 1e-2


def test_element_pairing_does_not_change_results():
    F, S, w0 = 8, 1560, 1560
    wl = Workload("wan-frames", 1, 2, 128, F, S, w0, 1.0)
    q, k, v = draw_qkv(wl, seed=4, device="cuda")
    host = radial.build_mask(F, S, w0)
    outs = []
    for t in (host.pairs, None):
        m = radial.Mask(host.row_ptr, host.col_idx, F, S, w0, t).to("cuda")
        outs.append(radial.attn_fwd(q, k, v, m, element=True))
    torch.cuda.synchronize()
    assert torch.equal(outs[0], outs[1])


def sampled_blocks(nb, seed):
    rng = np.random.default_rng(seed)
    picks = rng.choice(np.arange(2, nb - 2), size=3, replace=False)
    return sorted({0, 1, nb // 2, nb - 2, nb - 1, *picks.tolist()})


@pytest.mark.parametrize("key", ["wan", "hunyuan", "long4x"])
def test_element_parity_full_size_sampled(key):
    wl = WORKLOADS[key]
    q, k, v = draw_qkv(wl, seed=0, device="cuda")
    mask = radial.build_mask(wl.frames, wl.tokens_per_frame, wl.w0)
    o = radial.attn_fwd(q, k, v, mask.to("cuda"), element=True)
    torch.cuda.synchronize()
    blocks = sampled_blocks(wl.nb, seed=wl.n + 1)
    for h in sorted({0, wl.heads // 2, wl.heads - 1}):
        sl = (slice(None), slice(h, h + 1))
        ref, _ = oracle_element(q[sl], k[sl], v[sl], mask, wl.scale, query_blocks=blocks)
        rows = np.concatenate([np.arange(b * 128, min(wl.n, b * 128 + 128)) for b in blocks])
        check(o[sl], ref, rows=rows)
