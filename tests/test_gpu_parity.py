"""GPU parity: the HIP forward pass against the fp64 CPU oracle, on the same seeded inputs.

Bar: every checked output element within max-abs 2e-2 and mean-abs 2e-3 of the oracle.
The oracle sees the exact fp64 upcast of the bf16 tensors given to the GPU. Small shapes
are compared on every element. At full size the oracle walks its own CSR of the rule:
Wan is compared on every element of all 40 heads; HunyuanVideo and the 4x longer video
on every query block of one head and on sampled blocks of two more. out and lse start as
NaN, and every row of every head must come out finite.
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
    radial.lib()  # fail loudly if the library is missing


def f64(x):
    return x.detach().to("cpu", torch.float64).numpy()


def oracle_out(q, k, v, mask, scale, query_blocks=None):
    """The oracle over the same rule as `mask` (its own CSR, or its own all-active CSR for
    the dense mask)."""
    if mask.w0 == 2**31 - 1 and mask.frames == 1:
        rp, ci = ro.full_csr(mask.n)
    else:
        rp, ci = oracle_csr(mask.frames, mask.tokens_per_frame, mask.w0)
    return ro.attention(f64(q), f64(k), f64(v), rp, ci, scale, query_blocks=query_blocks)


def check(o_gpu, o_ref, rows=None, magnitude=1.0):
    """Max-abs / mean-abs bar. The output is a convex combination of V. Its error has
    two parts that both grow with the size of V: the final bf16 rounding (half an ulp,
    up to 2**-8 of the value) and the bf16 rounding of P inside the P V product (up to
    2**-8 of each weight, times |v_j - o|, so it reaches small outputs too: an
    elementwise bar of 2e-2 plus half an ulp of the reference fails at sigma = 4 by
    0.008). So for inputs drawn with sigma > 1 the absolute bar is scaled by
    `magnitude` = sigma. The pages' workloads all have sigma <= 1, and their bar is
    unscaled."""
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
    # 12 (batch, head)s: one XCD per head, four XCDs with two heads and four with one
    ("twelve-heads", 3, 4, 64, 5, 700, 200, 1.0),
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
    rp, ci = oracle_csr(wl.frames, wl.tokens_per_frame, wl.w0)
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


FULL = ["wan", "hunyuan", "long4x"]
# Wan's 40 heads are compared on every element, in groups of 8 heads per test (about
# half a minute of oracle time each on 16 host threads).
WAN_HEAD_GROUPS = [range(h, h + 8) for h in range(0, 40, 8)]

_full_cache = {}


def full_size_run(key):
    """The forward pass of a full-size workload, once per module: q, k, v drawn on the
    GPU, out and lse pre-filled with NaN (so a row the kernel skips stays NaN), and the
    oracle's own CSR of the rule. Only the latest workload is kept, to bound memory."""
    if key not in _full_cache:
        _full_cache.clear()
        torch.cuda.empty_cache()
        wl = WORKLOADS[key]
        q, k, v = draw_qkv(wl, seed=0, device="cuda")
        mask = radial.build_mask(wl.frames, wl.tokens_per_frame, wl.w0)
        rp, ci = oracle_csr(wl.frames, wl.tokens_per_frame, wl.w0)
        o = torch.full_like(q, float("nan"))
        lse = torch.full(q.shape[:3], float("nan"), dtype=torch.float32, device="cuda")
        radial.attn_fwd(q, k, v, mask.to("cuda"), out=o, lse=lse)
        torch.cuda.synchronize()
        _full_cache[key] = (wl, q, k, v, o, lse, mask, rp, ci)
    return _full_cache[key]


def compare_head(run, h, query_blocks=None):
    """Output and lse of head h (rows of `query_blocks`, or every row) against the
    oracle, which walks its own CSR."""
    wl, q, k, v, o, lse, _, rp, ci = run
    sl = (slice(None), slice(h, h + 1))
    ref, ref_lse = ro.attention(f64(q[sl]), f64(k[sl]), f64(v[sl]), rp, ci, wl.scale,
                                query_blocks=query_blocks)
    rows = None
    if query_blocks is not None:
        rows = np.concatenate([np.arange(b * 128, min(wl.n, b * 128 + 128))
                               for b in query_blocks])
    check(o[sl], ref, rows=rows)
    got_lse = f64(lse[sl])
    if rows is not None:
        got_lse, ref_lse = got_lse[..., rows], ref_lse[..., rows]
    assert np.abs(got_lse - ref_lse).max() < 1e-3


@pytest.mark.parametrize("key", FULL)
def test_full_size_mask_is_the_oracle_csr(key):
    _, _, _, _, _, _, mask, rp, ci = full_size_run(key)
    assert np.array_equal(mask.row_ptr.numpy(), rp)
    assert np.array_equal(mask.col_idx.numpy(), ci)


@pytest.mark.parametrize("key", FULL)
def test_full_size_every_row_written(key):
    """out and lse start as NaN: after one call every row of every (batch, head) must be
    finite, so no work item was skipped by the persistent scheduler."""
    _, _, _, _, o, lse, _, _, _ = full_size_run(key)
    assert bool(torch.isfinite(o).all())
    assert bool(torch.isfinite(lse).all())


@pytest.mark.parametrize("heads", WAN_HEAD_GROUPS,
                         ids=[f"heads{r.start}-{r.stop - 1}" for r in WAN_HEAD_GROUPS])
def test_wan_every_element(heads):
    run = full_size_run("wan")
    for h in heads:
        print(f"wan head {h}", flush=True)
        compare_head(run, h)


@pytest.mark.parametrize("key", ["hunyuan", "long4x"])
def test_full_size_one_head_every_block(key):
    """Every query block of the middle head against the oracle."""
    run = full_size_run(key)
    compare_head(run, run[0].heads // 2)


@pytest.mark.parametrize("key", ["hunyuan", "long4x"])
def test_full_size_sampled_blocks(key):
    """Sampled query blocks (the first two, the middle one, the last two with the ragged
    tail, and three seeded picks) of the first and the last head."""
    run = full_size_run(key)
    wl = run[0]
    blocks = sampled_blocks(wl.nb, seed=wl.n)
    for h in (0, wl.heads - 1):
        compare_head(run, h, query_blocks=blocks)


def test_many_work_items_full_output():
    """Small's shape with 64 heads: 2048 work items, eight per workgroup of the
    persistent grid on average, so the item loop, the per-XCD lists and the taking of
    items from other lists all run; every element against the oracle."""
    wl = Workload("small-64-heads", 1, 64, 64, 8, 1024, 512, 0.5)
    q, k, v = draw_qkv(wl, seed=9, device="cuda")
    mask = radial.build_mask(wl.frames, wl.tokens_per_frame, wl.w0)
    rp, ci = oracle_csr(wl.frames, wl.tokens_per_frame, wl.w0)
    for pairs in (True, False):
        m = mask if pairs else radial.Mask(mask.row_ptr, mask.col_idx, wl.frames,
                                           wl.tokens_per_frame, wl.w0)
        o = torch.full_like(q, float("nan"))
        lse = torch.full(q.shape[:3], float("nan"), dtype=torch.float32, device="cuda")
        radial.attn_fwd(q, k, v, m.to("cuda"), out=o, lse=lse)
        torch.cuda.synchronize()
        ref, ref_lse = ro.attention(f64(q), f64(k), f64(v), rp, ci, wl.scale)
        check(o, ref)
        assert np.abs(f64(lse) - ref_lse).max() < 1e-3


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
