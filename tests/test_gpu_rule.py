"""GPU tests of the on-the-fly mask (radial_attn_fwd_rule): the kernel derives each row's
key blocks from the rule instead of reading a CSR.

It visits the same key blocks in the same order as the CSR path, with the same
arithmetic, so output and lse must equal attn_fwd's on the built CSR bit for bit, for the
1-D and the grid distance, block and element semantics, with and without a pair table.
The CSR path is itself checked against the oracle elsewhere; one shape here is also
checked against the oracle directly (max-abs 2e-2, mean-abs 2e-3).
"""
import numpy as np
import pytest
import torch

import block_sparse_attention_radial_amd as radial
from block_sparse_attention_radial_amd.inputs import WORKLOADS, Workload, draw_qkv
from oracle import radial_oracle as ro

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    radial.lib()


def f64(x):
    return x.detach().to("cpu", torch.float64).numpy()


CASES = [
    # name, B, H, D, F, S, W0, grid_w, element, pairs
    ("wan-frames", 1, 2, 128, 21, 1560, 1560, None, False, False),
    ("narrow", 2, 2, 128, 6, 1000, 100, None, False, True),
    ("narrow-element", 1, 3, 64, 6, 300, 40, None, True, False),
    ("short-frames", 1, 2, 128, 12, 100, 37, None, False, False),   # frames under a block
    ("one-token-frames", 1, 1, 64, 300, 1, 1, None, False, False),
    ("one-frame", 1, 2, 128, 1, 5000, 1, None, False, True),        # diagonal blocks only
    ("huge-window", 1, 1, 128, 5, 333, 2**31 - 1, None, True, False),
    ("grid", 1, 2, 128, 6, 1000, 12, 50, False, False),
    ("grid-element", 1, 2, 128, 6, 1000, 12, 50, True, True),
    ("grid-rows-of-8", 2, 1, 64, 3, 200, 7, 8, True, False),
    ("grid-short-frames", 1, 2, 128, 9, 60, 4, 6, False, False),
]


@pytest.mark.parametrize("name,B,H,D,F,S,w0,gw,element,pairs", CASES, ids=[c[0] for c in CASES])
def test_rule_equals_csr_bitwise(name, B, H, D, F, S, w0, gw, element, pairs):
    wl = Workload(name, B, H, D, F, S, w0, 1.0, grid_w=gw)
    q, k, v = (x.cuda() for x in draw_qkv(wl, seed=21))
    csr = radial.build_mask(F, S, w0, pairs=pairs, grid_w=gw).to("cuda")
    rm = radial.rule_mask(F, S, w0, grid_w=gw, pairs=pairs).to("cuda")
    lse1 = torch.empty(B, H, wl.n, dtype=torch.float32, device="cuda")
    lse2 = torch.empty_like(lse1)
    o1 = radial.attn_fwd(q, k, v, csr, lse=lse1, element=element)
    o2 = radial.attn_fwd(q, k, v, rm, lse=lse2, element=element)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)
    assert torch.equal(lse1, lse2)


def test_rule_against_oracle():
    F, S, w0, D = 7, 500, 60, 128
    wl = Workload("oracle", 1, 2, D, F, S, w0, 1.0)
    q, k, v = draw_qkv(wl, seed=22)
    o = radial.attn_fwd(q.cuda(), k.cuda(), v.cuda(), radial.rule_mask(F, S, w0))
    torch.cuda.synchronize()
    rp, ci = ro.csr(ro.block_mask(F, S, w0))
    ref, _ = ro.attention(f64(q), f64(k), f64(v), rp, ci, wl.scale)
    err = np.abs(f64(o) - ref)
    assert err.max() <= 2e-2 and err.mean() <= 2e-3, (err.max(), err.mean())


def test_rule_full_size_wan_equals_csr():
    wl = WORKLOADS["wan"]
    q, k, v = draw_qkv(wl, seed=0, device="cuda", heads=range(4))
    csr = radial.build_mask(wl.frames, wl.tokens_per_frame, wl.w0).to("cuda")
    rm = radial.rule_mask(wl.frames, wl.tokens_per_frame, wl.w0, pairs=True).to("cuda")
    o1 = radial.attn_fwd(q, k, v, csr)
    o2 = radial.attn_fwd(q, k, v, rm)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)


def test_rule_autograd_matches_csr():
    wl = Workload("autograd", 1, 2, 128, 4, 1000, 200, 1.0)
    base = [x.cuda() for x in draw_qkv(wl, seed=23)]
    do = torch.randn_like(base[0])
    grads = []
    for mask in (radial.build_mask(4, 1000, 200).to("cuda"), radial.rule_mask(4, 1000, 200)):
        q, k, v = (x.clone().requires_grad_() for x in base)
        radial.attention(q, k, v, mask).backward(do)
        grads.append((q.grad, k.grad, v.grad))
    torch.cuda.synchronize()
    for a, b in zip(*grads):
        assert torch.equal(a, b)
