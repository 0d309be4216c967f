"""GPU parity: the HIP forward pass against the fp64 CPU oracle, on the same seeded inputs.

Bar: every checked output element within max-abs 2e-2 and mean-abs 2e-3 of the oracle.
The oracle sees the exact fp64 upcast of the bf16 tensors given to the GPU. Small shapes
are compared on every element. The full-size workloads are compared on sampled
query blocks: the first one, the ragged last one, and seeded picks between, for several
heads. The CPU oracle computes those blocks one by one.
"""
import numpy as np
import pytest
import torch

import block_sparse_attention_radial_amd as radial
from block_sparse_attention_radial_amd.inputs import WORKLOADS, Workload, draw_qkv
from oracle import radial_oracle as ro

pytestmark = pytest.mark.gpu

MAX_ABS, MEAN_ABS = 2e-2, 2e-3


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    radial.lib()  # fail loudly if the library is missing


def f64(x):
    return x.detach().to("cpu", torch.float64).numpy()


def oracle_out(q, k, v, mask, scale, query_blocks=None):
    rp, ci = mask.row_ptr.cpu().numpy(), mask.col_idx.cpu().numpy()
    return ro.attention(f64(q), f64(k), f64(v), rp, ci, scale, query_blocks=query_blocks)


def check(o_gpu, o_ref, rows=None, magnitude=1.0):
    """Max-abs / mean-abs bar. The output is a convex combination of V, and its error
    is dominated by the final bf16 rounding (relative 2**-9). So for inputs drawn with
    sigma > 1 the absolute bar is scaled by `magnitude` = sigma. The pages' workloads
    all have sigma <= 1, and their bar is unscaled."""
    got = f64(o_gpu)
    if rows is not None:
        got, o_ref = got[..., rows, :], o_ref[..., rows, :]
    err = np.abs(got - o_ref)
    assert np.isfinite(got).all()
    assert err.max() <= MAX_ABS * magnitude and err.mean() <= MEAN_ABS * magnitude, (
        err.max(), err.mean())
    return err.max(), err.mean()


SMALL = [
    # name, B, H, D, F, S, W0, sigma
    ("tiny", 1, 1, 64, 4, 256, 256, 1.0),
    ("small", 1, 8, 64, 8, 1024, 512, 0.5),
    ("ragged-sparse-d128", 2, 3, 128, 6, 1000, 100, 1.0),
    ("ragged-sparse-d64", 2, 3, 64, 6, 1000, 100, 1.0),
    ("ragged-half-d128", 1, 2, 128, 8, 1000, 334, 1.0),
    ("short-frames", 1, 2, 128, 12, 100, 37, 1.0),
    ("one-block", 1, 2, 128, 1, 100, 7, 1.0),
    ("single-token", 1, 1, 64, 1, 1, 1, 1.0),
    ("two-blocks-1-tail", 1, 1, 128, 1, 129, 1, 1.0),
    ("wide-values", 1, 2, 128, 4, 500, 300, 4.0),
]


@pytest.mark.parametrize("name,B,H,D,F,S,w0,sigma", SMALL, ids=[c[0] for c in SMALL])
def test_parity_small(name, B, H, D, F, S, w0, sigma):
    wl = Workload(name, B, H, D, F, S, w0, sigma)
    q, k, v = draw_qkv(wl, seed=0)
    mask = radial.build_mask(F, S, w0)
    dev = mask.to("cuda")
    lse = torch.empty(B, H, wl.n, dtype=torch.float32, device="cuda")
    o = radial.attn_fwd(q.cuda(), k.cuda(), v.cuda(), dev, lse=lse)
    torch.cuda.synchronize()
    ref, ref_lse = oracle_out(q, k, v, mask, wl.scale)
    check(o, ref, magnitude=max(1.0, sigma))
    assert np.abs(f64(lse) - ref_lse).max() < 1e-3 * max(1.0, sigma ** 2)


def test_scale_zero_is_mean_of_v_over_key_set():
    wl = Workload("s0", 1, 2, 128, 6, 1000, 100, 1.0)
    q, k, v = draw_qkv(wl, seed=1)
    mask = radial.build_mask(wl.frames, wl.tokens_per_frame, wl.w0)
    o = radial.attn_fwd(q.cuda(), k.cuda(), v.cuda(), mask.to("cuda"), scale=0.0)
    torch.cuda.synchronize()
    vv = f64(v)
    rp, ci = mask.row_ptr.numpy(), mask.col_idx.numpy()
    ref = np.empty_like(vv)
    for qb in range(mask.nb):
        keys = ro.row_keys(rp, ci, qb, wl.n)
        ref[..., qb * 128:(qb + 1) * 128, :] = vv[..., keys, :].mean(axis=-2, keepdims=True)
    check(o, ref)


def test_dense_mask_matches_oracle_dense():
    wl = Workload("dense", 1, 2, 128, 3, 700, 5, 1.0)
    q, k, v = draw_qkv(wl, seed=2)
    dense = radial.dense_mask(wl.n)
    o = radial.attn_fwd(q.cuda(), k.cuda(), v.cuda(), dense.to("cuda"))
    torch.cuda.synchronize()
    ref = torch.nn.functional.scaled_dot_product_attention(
        *(x.double() for x in (q, k, v))).numpy()
    check(o, ref)


def test_deterministic_and_layout_independent():
    wl = Workload("det", 1, 4, 128, 6, 1000, 100, 1.0)
    q, k, v = (x.cuda() for x in draw_qkv(wl, seed=3))
    mask = radial.build_mask(wl.frames, wl.tokens_per_frame, wl.w0).to("cuda")
    o1 = radial.attn_fwd(q, k, v, mask)
    o2 = radial.attn_fwd(q, k, v, mask)
    # The same tensors stored [B, n, H, D] and viewed as [B, H, n, D].
    qs, ks, vs = (x.transpose(1, 2).contiguous().transpose(1, 2) for x in (q, k, v))
    assert qs.stride() != q.stride()
    o3 = radial.attn_fwd(qs, ks, vs, mask)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)
    assert torch.equal(o1, o3.contiguous())


def test_out_of_range_columns_are_skipped():
    wl = Workload("skip", 1, 2, 64, 6, 1000, 100, 1.0)
    q, k, v = (x.cuda() for x in draw_qkv(wl, seed=4))
    mask = radial.build_mask(wl.frames, wl.tokens_per_frame, wl.w0)
    rp, ci = mask.row_ptr.clone(), mask.col_idx.tolist()
    # Insert an invalid column into row 3 and shift later rows.
    at = int(rp[4])
    ci.insert(at, mask.nb + 5)
    rp[4:] += 1
    bad = radial.Mask(rp, torch.tensor(ci, dtype=torch.int32), wl.frames, wl.tokens_per_frame,
                      wl.w0)
    o_ref = radial.attn_fwd(q, k, v, mask.to("cuda"))
    o_bad = radial.attn_fwd(q, k, v, bad.to("cuda"))
    torch.cuda.synchronize()
    assert torch.equal(o_ref, o_bad)


def sampled_blocks(nb, seed):
    rng = np.random.default_rng(seed)
    picks = {0, 1, nb // 2, nb - 2, nb - 1}
    picks.update(int(x) for x in rng.integers(0, nb, 3))
    return sorted(picks)


@pytest.mark.parametrize("key", ["wan", "hunyuan", "long4x"])
def test_parity_full_size_sampled(key):
    wl = WORKLOADS[key]
    q, k, v = draw_qkv(wl, seed=0, device="cuda")
    mask = radial.build_mask(wl.frames, wl.tokens_per_frame, wl.w0)
    o = radial.attn_fwd(q, k, v, mask.to("cuda"))
    torch.cuda.synchronize()
    blocks = sampled_blocks(wl.nb, seed=wl.n)
    for h in sorted({0, wl.heads // 2, wl.heads - 1}):
        sl = (slice(None), slice(h, h + 1))
        ref, _ = oracle_out(q[sl], k[sl], v[sl], mask, wl.scale, query_blocks=blocks)
        rows = np.concatenate([np.arange(b * 128, min(wl.n, b * 128 + 128)) for b in blocks])
        check(o[sl], ref, rows=rows)


def test_dense_full_size_sampled():
    # The same kernel with the all-active CSR (the dense baseline) at Wan shape.
    wl = WORKLOADS["wan"]
    q, k, v = draw_qkv(wl, seed=5, device="cuda", heads=range(2))
    dense = radial.dense_mask(wl.n)
    o = radial.attn_fwd(q, k, v, dense.to("cuda"))
    torch.cuda.synchronize()
    blocks = [0, 100, wl.nb - 1]
    ref, _ = oracle_out(q, k, v, dense, wl.scale, query_blocks=blocks)
    rows = np.concatenate([np.arange(b * 128, min(wl.n, b * 128 + 128)) for b in blocks])
    check(o, ref, rows=rows)
