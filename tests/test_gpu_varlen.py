"""GPU tests of the varlen forward: a packed batch of videos with different frame counts.

Each sample runs the same kernel arithmetic as attn_fwd on that sample alone, so the
packed result must equal the per-sample results bit for bit (block and element
semantics, with and without pair tables); the samples are also checked against the
fp64 oracle (bar as in test_gpu_parity: max-abs 2e-2, mean-abs 2e-3).
"""
import numpy as np
import pytest
import torch

import block_sparse_attention_radial_amd as radial
from oracle import radial_oracle as ro
from oracle_masks import oracle_csr

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    radial.lib()


def packed_inputs(total, H, D, seed, layout="thd"):
    g = torch.Generator(device="cuda").manual_seed(seed)
    if layout == "thd":  # [total, H, D] contiguous
        return [torch.randn(total, H, D, generator=g, device="cuda").to(torch.bfloat16)
                for _ in range(3)]
    # [H, total, D] storage viewed as [total, H, D]
    return [torch.randn(H, total, D, generator=g, device="cuda").to(torch.bfloat16).transpose(0, 1)
            for _ in range(3)]


CASES = [
    # frames, S, W0, H, D, pairs, element, layout
    ([21, 8, 3], 1560, 1560, 2, 128, True, False, "thd"),
    ([5, 12, 1, 7], 1000, 300, 3, 64, False, False, "thd"),
    ([6, 2, 9], 300, 40, 2, 128, True, True, "htd"),
    ([4], 256, 256, 1, 64, True, False, "thd"),
    # heads in multiples of 8 and of 4: the XCD groups of one and two XCDs per head
    ([5, 12, 1, 7], 1000, 300, 8, 64, True, False, "thd"),
    ([3, 9, 2], 600, 150, 4, 128, False, True, "htd"),
]


@pytest.mark.parametrize("frames,S,w0,H,D,pairs,element,layout", CASES)
def test_varlen_equals_per_sample(frames, S, w0, H, D, pairs, element, layout):
    masks = [radial.build_mask(f, S, w0, pairs=pairs) for f in frames]
    vm = radial.concat_masks(masks).to("cuda")
    total = sum(m.n for m in masks)
    q, k, v = packed_inputs(total, H, D, seed=len(frames) + D, layout=layout)
    lse = torch.empty(H, total, dtype=torch.float32, device="cuda")
    out = radial.attn_fwd_varlen(q, k, v, vm, lse=lse, element=element)
    t0 = 0
    for m in masks:
        sl = slice(t0, t0 + m.n)
        # The sample alone, as [1, H, n, D] views of the packed tensors.
        qs, ks, vs = (x[sl].permute(1, 0, 2).unsqueeze(0) for x in (q, k, v))
        ls = torch.empty(1, H, m.n, dtype=torch.float32, device="cuda")
        os = radial.attn_fwd(qs, ks, vs, m.to("cuda"), lse=ls, element=element)
        torch.cuda.synchronize()
        assert torch.equal(out[sl].permute(1, 0, 2).unsqueeze(0), os)
        assert torch.equal(lse[:, sl], ls[0])
        t0 += m.n


def test_varlen_parity_against_oracle():
    frames, S, w0, H, D = [6, 3, 11], 1000, 100, 2, 128
    masks = [radial.build_mask(f, S, w0) for f in frames]
    vm = radial.concat_masks(masks).to("cuda")
    total = sum(m.n for m in masks)
    q, k, v = packed_inputs(total, H, D, seed=21)
    out = radial.attn_fwd_varlen(q, k, v, vm)
    torch.cuda.synchronize()
    t0 = 0
    for m in masks:
        sl = slice(t0, t0 + m.n)
        f64 = lambda x: x[sl].permute(1, 0, 2).to("cpu", torch.float64).numpy()  # noqa: E731
        ref, _ = ro.attention(f64(q), f64(k), f64(v), *oracle_csr(m.frames, S, w0),
                              D ** -0.5)
        err = np.abs(f64(out) - ref)
        assert err.max() <= 2e-2 and err.mean() <= 2e-3, (err.max(), err.mean())
        t0 += m.n


def test_varlen_sixty_four_samples():
    """The largest batch the plan holds, with samples from one block up."""
    rng = np.random.default_rng(5)
    frames = [int(f) for f in rng.integers(1, 7, size=64)]
    S, w0, H, D = 120, 30, 2, 64
    masks = [radial.build_mask(f, S, w0) for f in frames]
    vm = radial.concat_masks(masks).to("cuda")
    total = sum(m.n for m in masks)
    q, k, v = packed_inputs(total, H, D, seed=64)
    lse = torch.empty(H, total, dtype=torch.float32, device="cuda")
    out = radial.attn_fwd_varlen(q, k, v, vm, lse=lse)
    torch.cuda.synchronize()
    t0 = 0
    for m in masks:
        sl = slice(t0, t0 + m.n)
        qs, ks, vs = (x[sl].permute(1, 0, 2).unsqueeze(0) for x in (q, k, v))
        ls = torch.empty(1, H, m.n, dtype=torch.float32, device="cuda")
        os_ = radial.attn_fwd(qs, ks, vs, m.to("cuda"), lse=ls)
        torch.cuda.synchronize()
        assert torch.equal(out[sl].permute(1, 0, 2).unsqueeze(0), os_)
        assert torch.equal(lse[:, sl], ls[0])
        t0 += m.n


def test_varlen_rejects_a_sixty_fifth_sample():
    masks = [radial.build_mask(1, 128, 10) for _ in range(65)]
    vm = radial.concat_masks(masks).to("cuda")
    q, k, v = packed_inputs(65 * 128, 1, 64, seed=65)
    with pytest.raises(radial.RadialError):
        radial.attn_fwd_varlen(q, k, v, vm)


BWD_CASES = [
    # frames, S, W0, grid_w, H, D, element
    ([7, 3, 11], 300, 40, None, 2, 128, False),
    ([5, 2, 9], 300, 40, None, 2, 64, True),
    ([4, 6], 200, 9, 8, 1, 128, True),
    # the Wan-shaped batch at full size, 8 heads (the forward's XCD groups of one XCD)
    ([21, 16, 11, 5], 1560, 1560, None, 8, 128, False),
]


@pytest.mark.parametrize("frames,S,w0,gw,H,D,element", BWD_CASES)
def test_varlen_backward_equals_per_sample(frames, S, w0, gw, H, D, element):
    masks = [radial.build_mask(f, S, w0, grid_w=gw) for f in frames]
    vm = radial.concat_masks(masks).to("cuda")
    total = sum(m.n for m in masks)
    q, k, v = packed_inputs(total, H, D, seed=31 + D)
    g = torch.Generator(device="cuda").manual_seed(32)
    do = torch.randn(q.shape, generator=g, device="cuda").to(torch.bfloat16)
    lse = torch.empty(H, total, dtype=torch.float32, device="cuda")
    o = radial.attn_fwd_varlen(q, k, v, vm, lse=lse, element=element)
    grads = radial.attn_bwd_varlen(q, k, v, o, do, lse, vm, element=element)
    torch.cuda.synchronize()
    t0 = 0
    for m in masks:
        sl = slice(t0, t0 + m.n)
        view = lambda x: x[sl].permute(1, 0, 2).unsqueeze(0)  # noqa: E731
        md = m.to("cuda")
        ls = torch.empty(1, H, m.n, dtype=torch.float32, device="cuda")
        os_ = radial.attn_fwd(view(q), view(k), view(v), md, lse=ls, element=element)
        ref = radial.attn_bwd(view(q), view(k), view(v), os_, view(do), ls, md,
                              element=element)
        torch.cuda.synchronize()
        for got, r in zip(grads, ref):
            assert torch.equal(view(got), r)
        t0 += m.n


def test_varlen_backward_against_oracle():
    frames, S, w0, H, D = [4, 2], 500, 60, 2, 128
    masks = [radial.build_mask(f, S, w0) for f in frames]
    vm = radial.concat_masks(masks).to("cuda")
    total = sum(m.n for m in masks)
    q, k, v = (x.requires_grad_() for x in packed_inputs(total, H, D, seed=33))
    g = torch.Generator(device="cuda").manual_seed(34)
    do = torch.randn(q.shape, generator=g, device="cuda").to(torch.bfloat16)
    radial.attention_varlen(q, k, v, vm).backward(do)
    torch.cuda.synchronize()
    t0 = 0
    for m in masks:
        sl = slice(t0, t0 + m.n)
        f64 = lambda x: x.detach()[sl].permute(1, 0, 2).to("cpu", torch.float64).numpy()  # noqa: E731
        ref = ro.attention_backward(f64(q), f64(k), f64(v), f64(do),
                                    *oracle_csr(m.frames, S, w0), D ** -0.5)
        for got, r in zip((q.grad, k.grad, v.grad), ref):
            err = np.abs(f64(got) - r)
            assert err.max() <= 2e-2 * np.abs(r).max() and err.mean() <= 5e-3 * np.abs(r).mean()
        t0 += m.n


RULE_CASES = [
    # frames, S, W0, grid_w, H, D, element, pairs
    ([21, 8, 3], 1560, 1560, None, 2, 128, False, True),
    ([5, 12, 1, 7], 1000, 300, None, 3, 64, True, False),
    ([6, 2, 9], 300, 40, 20, 2, 128, True, True),
    ([3, 40], 100, 37, None, 1, 64, False, False),  # frames shorter than a block
]


@pytest.mark.parametrize("frames,S,w0,gw,H,D,element,pairs", RULE_CASES)
def test_varlen_rule_equals_varlen_csr(frames, S, w0, gw, H, D, element, pairs):
    masks = [radial.build_mask(f, S, w0, pairs=pairs, grid_w=gw) for f in frames]
    vm = radial.concat_masks(masks)
    rm = radial.VarlenRuleMask(frames, S, w0, gw or 0, vm.pairs, vm.npairs)
    total = sum(m.n for m in masks)
    q, k, v = packed_inputs(total, H, D, seed=50 + D)
    lse1 = torch.empty(H, total, dtype=torch.float32, device="cuda")
    lse2 = torch.empty_like(lse1)
    o1 = radial.attn_fwd_varlen(q, k, v, vm.to("cuda"), lse=lse1, element=element)
    o2 = radial.attn_fwd_varlen(q, k, v, rm.to("cuda"), lse=lse2, element=element)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)
    assert torch.equal(lse1, lse2)


def test_varlen_rule_autograd_matches_csr():
    frames, S, w0, H, D = [4, 2, 5], 300, 40, 2, 128
    vm = radial.build_varlen_mask(frames, S, w0).to("cuda")
    rm = radial.VarlenRuleMask(frames, S, w0)
    total = sum(f * S for f in frames)
    base = packed_inputs(total, H, D, seed=60)
    g = torch.Generator(device="cuda").manual_seed(61)
    do = torch.randn(base[0].shape, generator=g, device="cuda").to(torch.bfloat16)
    grads = []
    for mask in (vm, rm):
        q, k, v = (x.clone().requires_grad_() for x in base)
        radial.attention_varlen(q, k, v, mask).backward(do)
        grads.append((q.grad, k.grad, v.grad))
    torch.cuda.synchronize()
    for a, b in zip(*grads):
        assert torch.equal(a, b)
