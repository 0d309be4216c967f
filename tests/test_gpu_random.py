"""A seeded sweep over the forward's and backward's options against the oracle.

Each case draws a video shape (frames, frame length, W0, 1-D or grid distance), a
semantics (block or element), a pair table or none, CSR or on-the-fly mask, head_dim,
batch, heads and a storage layout, then checks the GPU output and lse against the fp64
oracle (max-abs 2e-2, mean-abs 2e-3, lse 1e-3) and, on every third case, the gradients
(relative bars as in test_gpu_backward). Element masking through a CSR is also run from
the mask's element table, which must give the same bits. Shapes stay small enough for the
oracle.
"""
import numpy as np
import pytest
import torch

import block_sparse_attention_radial_amd as radial
from block_sparse_attention_radial_amd.inputs import Workload, draw_qkv
from oracle import radial_oracle as ro
from oracle_masks import oracle_csr

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    radial.lib()


def f64(x):
    return x.detach().to("cpu", torch.float64).numpy()


def draw_case(seed):
    rng = np.random.default_rng(seed)
    element = bool(rng.integers(2))
    grid = bool(rng.integers(2))
    while True:
        F = int(rng.integers(1, 9))
        if grid:
            gh, gw = int(rng.integers(2, 30)), int(rng.integers(2, 60))
            S = gh * gw
        else:
            gw, S = None, int(rng.integers(1, 1200))
        if element and S < 128:
            continue
        if 1 <= F * S <= 4000:
            break
    reach = (gh + gw) if grid else S
    w0 = int(rng.integers(1, 2 * reach + 2))
    return dict(F=F, S=S, w0=w0, gw=gw, element=element, pairs=bool(rng.integers(2)),
                rule=bool(rng.integers(2)), D=int(rng.choice([64, 128])),
                B=int(rng.integers(1, 3)), H=int(rng.integers(1, 3)),
                bnhd=bool(rng.integers(2)))


@pytest.mark.parametrize("seed", range(48))
def test_random_case_against_oracle(seed):
    c = draw_case(1000 + seed)
    wl = Workload(f"random{seed}", c["B"], c["H"], c["D"], c["F"], c["S"], c["w0"], 1.0,
                  grid_w=c["gw"])
    q, k, v = draw_qkv(wl, seed=seed)
    if c["bnhd"]:  # [B, n, H, D] storage viewed as [B, H, n, D]
        q, k, v = (x.transpose(1, 2).contiguous().transpose(1, 2) for x in (q, k, v))
    mask = radial.build_mask(c["F"], c["S"], c["w0"], pairs=c["pairs"], grid_w=c["gw"])
    md = (radial.rule_mask(c["F"], c["S"], c["w0"], grid_w=c["gw"], pairs=c["pairs"])
          if c["rule"] else mask).to("cuda")
    qc, kc, vc = (x.cuda() for x in (q, k, v))
    lse = torch.empty(c["B"], c["H"], wl.n, dtype=torch.float32, device="cuda")
    o = radial.attn_fwd(qc, kc, vc, md, lse=lse, element=c["element"])
    torch.cuda.synchronize()
    rule = ((c["S"], c["w0"]) + ((c["gw"],) if c["gw"] else ())) if c["element"] else None
    rp, ci = oracle_csr(c["F"], c["S"], c["w0"], c["gw"])
    ref, ref_lse = ro.attention(f64(q), f64(k), f64(v), rp, ci, wl.scale, element=rule)
    err = np.abs(f64(o) - ref)
    assert np.isfinite(f64(o)).all()
    assert err.max() <= 2e-2 and err.mean() <= 2e-3, (c, err.max(), err.mean())
    assert np.abs(f64(lse) - ref_lse).max() < 1e-3, c
    table = None
    if c["element"] and not c["rule"]:
        table = radial.Mask(**{**md.__dict__, "element_table": None}).with_element_table()
        lse_t = torch.empty_like(lse)
        o_t = radial.attn_fwd(qc, kc, vc, table, lse=lse_t, element=True)
        torch.cuda.synchronize()
        assert torch.equal(o_t.view(torch.int16), o.view(torch.int16)), c
        assert torch.equal(lse_t.view(torch.int32), lse.view(torch.int32)), c
    if seed % 3:
        return
    g = torch.Generator().manual_seed(seed + 7)
    do = torch.randn(q.shape, generator=g).to(torch.bfloat16)
    if c["bnhd"]:
        do = do.transpose(1, 2).contiguous().transpose(1, 2)
    grads = radial.attn_bwd(qc, kc, vc, o, do.cuda(), lse, md, element=c["element"])
    if table is not None:
        for a, b in zip(grads, radial.attn_bwd(qc, kc, vc, o, do.cuda(), lse, table,
                                               element=True)):
            assert torch.equal(a.view(torch.int16), b.view(torch.int16)), c
    torch.cuda.synchronize()
    refs = ro.attention_backward(f64(q), f64(k), f64(v), f64(do), rp, ci, wl.scale,
                                 element=rule)
    for got, r in zip(grads, refs):
        got = f64(got)
        e = np.abs(got - r)
        assert np.isfinite(got).all()
        assert e.max() <= 2e-2 * np.abs(r).max() and e.mean() <= 5e-3 * np.abs(r).mean(), c
