"""Pins for the CPU oracle, each checked against something other than the oracle itself.

* Brute force. Pure-Python loops over every (query, key) pair, with the window taken as
  an exact rational W0 / 2**floor(math.log2(d + 1)) (fractions.Fraction).
* Closed forms. Hand-derived values, the total allowed-element count from a counting
  identity, and the worked block at Wan shape.
* Invariants. Diagonal allowed, symmetry, frame-Toeplitz structure, monotone in W0,
  no empty rows, sub-quadratic element growth.
* Library routines. torch's scaled_dot_product_attention in fp64 and
  scipy.special.logsumexp.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import radial_oracle as ro

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# --------------------------------------------------------------------------------------
# Brute-force helpers (pure Python; no oracle code)
# --------------------------------------------------------------------------------------

def bf_allowed(t_q, t_k, S, w0):
    fq, sq = divmod(t_q, S)
    fk, sk = divmod(t_k, S)
    d = abs(fq - fk)
    window = Fraction(w0, 2 ** math.floor(math.log2(d + 1)))
    return abs(sq - sk) < window


def bf_block_mask(F, S, w0, block):
    n = F * S
    nb = -(-n // block)
    out = [[False] * nb for _ in range(nb)]
    for i in range(n):
        for j in range(n):
            if bf_allowed(i, j, S, w0):
                out[i // block][j // block] = True
    return np.array(out, dtype=bool)


def bf_key_set(F, S, w0, block, qb):
    bm = bf_block_mask(F, S, w0, block)
    n = F * S
    return [j for j in range(n) if bm[qb][j // block]]


# --------------------------------------------------------------------------------------
# Element rule
# --------------------------------------------------------------------------------------

def test_band_hand_values():
    # floor(log2(d + 1)) for d = 0..7, worked by hand.
    assert ro.band(np.arange(8)).tolist() == [0, 1, 1, 2, 2, 2, 2, 3]


def test_band_matches_bit_length_and_log2():
    d = np.arange(0, 200_000)
    got = ro.band(d)
    assert all(int(g) == (int(x) + 1).bit_length() - 1 for g, x in zip(got[::997], d[::997]))
    # every power-of-two boundary, where a rounding slip would show
    for p in range(1, 40):
        x = 2 ** p
        assert int(ro.band(x - 1)) == p and int(ro.band(x - 2)) == p - 1
        assert math.floor(math.log2(x)) == p


SHAPES_BF = [  # (F, S, W0)
    (1, 40, 7), (2, 30, 1), (3, 17, 17), (4, 20, 19), (5, 12, 13), (6, 9, 33),
    (3, 25, 49), (4, 16, 46), (6, 11, 1000),
]


@pytest.mark.parametrize("F,S,w0", SHAPES_BF)
def test_element_mask_vs_exact_rational_bruteforce(F, S, w0):
    m = ro.element_mask(F, S, w0)
    n = F * S
    bf = np.array([[bf_allowed(i, j, S, w0) for j in range(n)] for i in range(n)])
    assert np.array_equal(m, bf)


def test_element_mask_edge_windows():
    # W0 in {1, S - 1, S, S + 1, (S - 1) * 2**k + 1}: the edges of the strict "<" test.
    F, S = 5, 13
    n = F * S
    for w0 in (1, S - 1, S, S + 1, (S - 1) * 2 + 1, (S - 1) * 4 + 1, (S - 1) * 4):
        m = ro.element_mask(F, S, w0)
        bf = np.array([[bf_allowed(i, j, S, w0) for j in range(n)] for i in range(n)])
        assert np.array_equal(m, bf), w0


def test_single_frame_is_sliding_window():
    # With one frame every pair has d = 0, so the rule is the band |i - j| < W0.
    S, w0 = 300, 37
    i = np.arange(S)
    assert np.array_equal(ro.element_mask(1, S, w0), np.abs(i[:, None] - i[None, :]) < w0)


def test_element_dense_iff_window_covers_frame():
    # Largest band is floor(log2 F) at d = F - 1; dense iff (S - 1) * 2**that < W0.
    for F, S in [(4, 10), (5, 10), (8, 7), (9, 7)]:
        top = 2 ** math.floor(math.log2(F))
        assert ro.element_mask(F, S, (S - 1) * top + 1).all()
        assert not ro.element_mask(F, S, (S - 1) * top).all()


@pytest.mark.parametrize("F,S,w0", [(6, 40, 25), (5, 33, 70), (8, 16, 9)])
def test_element_invariants(F, S, w0):
    m = ro.element_mask(F, S, w0)
    n = F * S
    assert m.diagonal().all()                      # every query sees itself
    assert np.array_equal(m, m.T)                  # symmetric
    assert m.any(axis=1).all()                     # no empty row
    # frame-Toeplitz: shifting both frames by c changes nothing
    blocks = m.reshape(F, S, F, S)
    for c in range(1, F):
        assert np.array_equal(blocks[c:, :, c:, :], blocks[:-c, :, :-c, :])
    # monotone in W0
    assert (ro.element_mask(F, S, w0 + 1) | ~m).all()
    assert n == m.shape[0]


# --------------------------------------------------------------------------------------
# Block reduction
# --------------------------------------------------------------------------------------

@pytest.mark.parametrize("F,S,w0,block", [
    (3, 10, 4, 8), (4, 7, 6, 8), (2, 13, 13, 8), (5, 6, 20, 4),
])
def test_block_mask_vs_bruteforce(F, S, w0, block):
    assert np.array_equal(ro.block_mask(F, S, w0, block), bf_block_mask(F, S, w0, block))


@pytest.mark.parametrize("F,S,w0,block", [
    (4, 256, 256, 128),      # Tiny shape
    (6, 100, 10, 32),        # S < block: blocks straddle several frames
    (6, 1000, 100, 128),     # ragged last block
    (8, 1000, 334, 128),
    (3, 777, 1555, 128),
    (7, 50, 3, 16),
    (16, 60, 200, 64),
])
def test_block_counts_vs_element_reduction(F, S, w0, block):
    counts = ro.block_counts(F, S, w0, block)
    assert np.array_equal(counts, ro.block_counts_from_elements(ro.element_mask(F, S, w0), block))


def closed_form_count(F, S, w0):
    """Allowed pairs: sum over frame distances d (F pairs at d = 0, 2(F - d) at d > 0)
    of the in-frame pairs with |ds| * 2**band(d) < W0. There are S pairs with ds = 0 and
    2(S - ds) with each ds > 0."""
    total = 0
    for d in range(F):
        mult = F if d == 0 else 2 * (F - d)
        k = (d + 1).bit_length() - 1
        inframe = sum((S if ds == 0 else 2 * (S - ds)) for ds in range(S) if ds * 2 ** k < w0)
        total += mult * inframe
    return total


@pytest.mark.parametrize("F,S,w0", [(4, 256, 256), (8, 1024, 512), (21, 1560, 1560),
                                    (6, 1000, 100), (84, 1560, 1560)])
def test_total_count_closed_form(F, S, w0):
    assert int(ro.block_counts(F, S, w0).sum()) == closed_form_count(F, S, w0)


def test_wan_worked_block():
    """Block (query 1, key 243) at Wan shape (S = W0 = 1560).

    Query block 1 is tokens 128..255, all in frame 0. Key block 243 is tokens
    31104..31231, which is frame 19, s = 1464..1559, and frame 20, s = 0..31. For frame
    20, d = 20 and floor(log2 21) = 4, so a pair is allowed iff 16 * |ds| < 1560, i.e.
    |ds| <= 97. The smallest |ds| is 128 - 31 = 97, reached only by (s_q = 128,
    s_k = 31). For frame 19 the smallest |ds| is 1464 - 255 = 1209, which is far too
    large. So exactly one element is allowed and the block is active. Reading W0/2**k
    as an integer shift (1560 >> 4 = 97, and 97 < 97 is false) would drop this block.
    """
    counts = ro.block_counts(21, 1560, 1560)
    assert counts[1, 243] == 1
    assert ro.allowed(0, 128, 20, 31, 1560) and not ro.allowed(0, 128, 20, 30, 1560)


def test_block_invariants_and_tiny_block_dense():
    for F, S, w0 in [(8, 1024, 512), (21, 1560, 1560), (6, 1000, 100)]:
        bm = ro.block_mask(F, S, w0)
        assert np.array_equal(bm, bm.T)
        assert bm.diagonal().all()
    # Tiny: 77% of elements allowed, yet every 128 x 128 block holds one.
    bm = ro.block_mask(4, 256, 256)
    assert bm.all() and bm.shape == (8, 8)


@pytest.mark.slow
def test_growth_is_subquadratic():
    # Wan spatial shape: elements grow by < 4x per doubling of frames, and the ratio falls.
    S = w0 = 1560
    totals = [closed_form_count(F, S, w0) for F in (2, 4, 8, 16, 32, 64)]
    ratios = [b / a for a, b in zip(totals, totals[1:])]
    assert all(r < 4 for r in ratios)
    assert all(b < a for a, b in zip(ratios, ratios[1:]))
    blocks = [int(ro.block_mask(F, S, w0).sum()) for F in (2, 4, 8, 16)]
    assert all(b / a < 4 for a, b in zip(blocks, blocks[1:]))


def test_csr_roundtrip():
    bm = ro.block_mask(6, 1000, 100)
    row_ptr, col_idx = ro.csr(bm)
    assert row_ptr.dtype == np.int32 and col_idx.dtype == np.int32
    assert row_ptr[0] == 0 and row_ptr[-1] == bm.sum()
    back = np.zeros_like(bm)
    for r in range(bm.shape[0]):
        cols = col_idx[row_ptr[r]:row_ptr[r + 1]]
        assert np.all(np.diff(cols) > 0)
        back[r, cols] = True
    assert np.array_equal(back, bm)


def test_csr_nonsymmetric_vs_loops():
    # A random, non-symmetric mask (with an empty row) against a plain loop build.
    rng = np.random.default_rng(3)
    bm = rng.random((37, 41)) < 0.3
    bm[5] = False
    row_ptr, col_idx = ro.csr(bm)
    rp, ci = [0], []
    for r in range(bm.shape[0]):
        for c in range(bm.shape[1]):
            if bm[r, c]:
                ci.append(c)
        rp.append(len(ci))
    assert row_ptr.tolist() == rp and col_idx.tolist() == ci


def test_golden_mask_summaries():
    """Block-mask summaries stored by tests/golden/make_golden.py (which calls only the
    oracle) must still be reproduced, so a later edit of the oracle cannot silently move
    the masks."""
    with open(os.path.join(GOLDEN, "masks.json")) as f:
        gold = json.load(f)
    for case in gold["cases"]:
        if case["n"] > 40_000:
            continue  # the large ones are covered by the slow test below
        bm = ro.block_mask(case["frames"], case["tokens_per_frame"], case["w0"],
                           grid_w=case.get("grid_w"))
        row_ptr, col_idx = ro.csr(bm)
        assert int(row_ptr[-1]) == case["nnz"]
        assert ro_digest(row_ptr, col_idx) == case["sha256"]


@pytest.mark.slow
def test_golden_mask_summaries_large():
    with open(os.path.join(GOLDEN, "masks.json")) as f:
        gold = json.load(f)
    for case in gold["cases"]:
        if case["n"] <= 40_000:
            continue
        bm = ro.block_mask(case["frames"], case["tokens_per_frame"], case["w0"],
                           grid_w=case.get("grid_w"))
        row_ptr, col_idx = ro.csr(bm)
        assert int(row_ptr[-1]) == case["nnz"]
        assert ro_digest(row_ptr, col_idx) == case["sha256"]


def ro_digest(row_ptr, col_idx):
    import hashlib
    h = hashlib.sha256()
    h.update(np.asarray(row_ptr, dtype="<i4").tobytes())
    h.update(np.asarray(col_idx, dtype="<i4").tobytes())
    return h.hexdigest()


# --------------------------------------------------------------------------------------
# Attention
# --------------------------------------------------------------------------------------

def rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def test_dense_mask_matches_torch_sdpa():
    n, D = 300, 32
    q, k, v = (rand((2, 3, n, D), s) for s in (1, 2, 3))
    rp, ci = ro.full_csr(n, 128)
    o, _ = ro.attention(q, k, v, rp, ci, scale=0.3)
    ref = torch.nn.functional.scaled_dot_product_attention(
        *(torch.from_numpy(x) for x in (q, k, v)), scale=0.3).numpy()
    assert np.abs(o - ref).max() < 1e-12


def test_tiny_block_dense_equals_dense():
    F, S, w0, D = 4, 256, 256, 64
    n = F * S
    q, k, v = (rand((1, 1, n, D), s) for s in (4, 5, 6))
    rp, ci = ro.csr(ro.block_mask(F, S, w0))
    o, _ = ro.attention(q, k, v, rp, ci, scale=D ** -0.5)
    ref = torch.nn.functional.scaled_dot_product_attention(
        *(torch.from_numpy(x) for x in (q, k, v))).numpy()
    assert np.abs(o - ref).max() < 1e-12


def test_bruteforce_rows_fsum():
    F, S, w0, block, D = 3, 10, 4, 8, 5
    n = F * S
    q, k, v = (rand((n, D), s) for s in (7, 8, 9))
    rp, ci = ro.csr(ro.block_mask(F, S, w0, block))
    o, lse = ro.attention(q, k, v, rp, ci, scale=0.7, block=block)
    for i in range(n):
        keys = bf_key_set(F, S, w0, block, i // block)
        x = [0.7 * math.fsum(q[i, c] * k[j, c] for c in range(D)) for j in keys]
        mx = max(x)
        p = [math.exp(t - mx) for t in x]
        l = math.fsum(p)
        for c in range(D):
            ref = math.fsum(pj * v[j, c] for pj, j in zip(p, keys)) / l
            assert abs(o[i, c] - ref) < 1e-12
        assert abs(lse[i] - (mx + math.log(l))) < 1e-12


def test_scale_zero_is_mean_over_key_set():
    F, S, w0, block, D = 4, 9, 5, 8, 6
    n = F * S
    q, k, v = (rand((n, D), s) for s in (10, 11, 12))
    rp, ci = ro.csr(ro.block_mask(F, S, w0, block))
    o, _ = ro.attention(q, k, v, rp, ci, scale=0.0, block=block)
    for qb in range(-(-n // block)):
        keys = bf_key_set(F, S, w0, block, qb)
        mean = v[keys].mean(axis=0)
        for i in range(qb * block, min(n, qb * block + block)):
            assert np.abs(o[i] - mean).max() < 1e-12


def test_constant_v_and_convexity():
    F, S, w0 = 6, 100, 10
    n = F * S
    rp, ci = ro.csr(ro.block_mask(F, S, w0))
    q, k = rand((n, 16), 13), rand((n, 16), 14)
    o, _ = ro.attention(q, k, np.full((n, 16), 0.375), rp, ci, scale=0.25)
    assert np.abs(o - 0.375).max() < 1e-14
    v = rand((n, 16), 15)
    o, _ = ro.attention(q, k, v, rp, ci, scale=0.25)
    assert (o <= v.max(axis=0) + 1e-12).all() and (o >= v.min(axis=0) - 1e-12).all()


def test_one_hot_v_recovers_probabilities():
    # With V = identity (n = D), o[i, j] is the softmax weight of key j for query i:
    # zero exactly off the key set, rows summing to one.
    F, S, w0, block = 4, 8, 3, 8
    n = F * S
    rp, ci = ro.csr(ro.block_mask(F, S, w0, block))
    q, k = rand((n, 4), 16), rand((n, 4), 17)
    o, _ = ro.attention(q, k, np.eye(n), rp, ci, scale=1.0, block=block)
    for i in range(n):
        keys = set(bf_key_set(F, S, w0, block, i // block))
        assert set(np.nonzero(o[i])[0].tolist()) == keys
        assert abs(o[i].sum() - 1.0) < 1e-13


def test_lse_matches_scipy():
    from scipy.special import logsumexp
    F, S, w0 = 6, 100, 10
    n = F * S
    rp, ci = ro.csr(ro.block_mask(F, S, w0))
    q, k, v = (rand((n, 8), s) for s in (18, 19, 20))
    _, lse = ro.attention(q, k, v, rp, ci, scale=0.5)
    for i in range(0, n, 37):
        keys = ro.row_keys(rp, ci, i // 128, n)
        assert abs(lse[i] - logsumexp(0.5 * (k[keys] @ q[i]))) < 1e-12


def test_ragged_padding_keys_excluded():
    # n = 6000 is not a multiple of 128; the last block's 16 padding keys never count.
    n = 6000
    rp, ci = ro.full_csr(n, 128)
    keys = ro.row_keys(rp, ci, 0, n)
    assert keys.max() == n - 1 and len(keys) == n


# --------------------------------------------------------------------------------------
# Element semantics (the rule applied inside the active blocks)
# --------------------------------------------------------------------------------------

def test_element_semantics_bruteforce_rows_fsum():
    """Exact-rational rule and math.fsum per row, against the oracle's element option."""
    F, S, w0, block, D = 3, 10, 4, 8, 5
    n = F * S
    q, k, v = (rand((n, D), s) for s in (31, 32, 33))
    rp, ci = ro.csr(ro.block_mask(F, S, w0, block))
    o, lse = ro.attention(q, k, v, rp, ci, scale=0.7, block=block, element=(S, w0))
    for i in range(n):
        keys = [j for j in range(n) if bf_allowed(i, j, S, w0)]
        x = [0.7 * math.fsum(q[i, c] * k[j, c] for c in range(D)) for j in keys]
        mx = max(x)
        p = [math.exp(t - mx) for t in x]
        l = math.fsum(p)
        for c in range(D):
            ref = math.fsum(pj * v[j, c] for pj, j in zip(p, keys)) / l
            assert abs(o[i, c] - ref) < 1e-12
        assert abs(lse[i] - (mx + math.log(l))) < 1e-12


def test_element_semantics_single_frame_is_torch_sliding_window():
    """F = 1: the rule is |i - j| < W0, a banded mask built here directly, fed to torch's
    scaled_dot_product_attention (fp64, CPU)."""
    n, w0, D = 700, 45, 16
    q, k, v = (rand((2, n, D), s) for s in (34, 35, 36))
    rp, ci = ro.csr(ro.block_mask(1, n, w0))
    o, _ = ro.attention(q, k, v, rp, ci, scale=0.3, element=(n, w0))
    i = np.arange(n)
    band_mask = torch.from_numpy(np.abs(i[:, None] - i[None, :]) < w0)
    ref = torch.nn.functional.scaled_dot_product_attention(
        *(torch.from_numpy(x) for x in (q, k, v)), attn_mask=band_mask, scale=0.3).numpy()
    assert np.abs(o - ref).max() < 1e-12


def test_element_semantics_element_dense_window_is_dense():
    """(S - 1) * 2**floor(log2 F) < W0 allows every pair: element semantics is dense."""
    F, S, D = 5, 60, 8
    w0 = (S - 1) * 4 + 1
    n = F * S
    q, k, v = (rand((n, D), s) for s in (37, 38, 39))
    rp, ci = ro.csr(ro.block_mask(F, S, w0))
    o, _ = ro.attention(q, k, v, rp, ci, scale=0.4, element=(S, w0))
    ref = torch.nn.functional.scaled_dot_product_attention(
        *(torch.from_numpy(x)[None] for x in (q, k, v)), scale=0.4)[0].numpy()
    assert np.abs(o - ref).max() < 1e-12


def test_element_semantics_scale_zero_is_mean_over_allowed_keys():
    F, S, w0, D = 4, 150, 40, 6
    n = F * S
    q, k, v = (rand((n, D), s) for s in (40, 41, 42))
    rp, ci = ro.csr(ro.block_mask(F, S, w0))
    o, _ = ro.attention(q, k, v, rp, ci, scale=0.0, element=(S, w0))
    for i in range(0, n, 23):
        keys = [j for j in range(n) if bf_allowed(i, j, S, w0)]
        assert np.abs(o[i] - v[keys].mean(axis=0)).max() < 1e-12


def test_element_semantics_removes_entries_block_semantics_keeps():
    """With a narrow window the two semantics differ, and element semantics never
    reaches a key that block semantics does not."""
    F, S, w0, D = 4, 256, 40, 8
    n = F * S
    q, k = rand((n, D), 43), rand((n, D), 44)
    rp, ci = ro.csr(ro.block_mask(F, S, w0))
    o_blk, _ = ro.attention(q, k, np.eye(n)[:, :n], rp, ci, scale=1.0)
    o_el, _ = ro.attention(q, k, np.eye(n)[:, :n], rp, ci, scale=1.0, element=(S, w0))
    assert np.abs(o_blk - o_el).max() > 1e-3
    assert ((o_el > 0) <= (o_blk > 0)).all()
    for i in range(0, n, 41):
        assert set(np.nonzero(o_el[i])[0].tolist()) == {
            j for j in range(n) if bf_allowed(i, j, S, w0)}


# --------------------------------------------------------------------------------------
# Backward (dq, dk, dv)
# --------------------------------------------------------------------------------------

def test_backward_matches_finite_differences():
    """Central differences of L = sum(o * do) in every input entry, on a tiny shape
    with a sparse block mask."""
    F, S, w0, block, D = 3, 6, 2, 4, 3
    n = F * S
    q, k, v, do = (rand((n, D), s) for s in (51, 52, 53, 54))
    rp, ci = ro.csr(ro.block_mask(F, S, w0, block))
    dq, dk, dv = ro.attention_backward(q, k, v, do, rp, ci, scale=0.8, block=block)

    def loss(q_, k_, v_):
        o, _ = ro.attention(q_, k_, v_, rp, ci, scale=0.8, block=block)
        return math.fsum((o * do).ravel())

    h = 1e-6
    for name, x, grad in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            args_p = {"q": q, "k": k, "v": v, name: xp}
            args_m = {"q": q, "k": k, "v": v, name: xm}
            num = (loss(args_p["q"], args_p["k"], args_p["v"])
                   - loss(args_m["q"], args_m["k"], args_m["v"])) / (2 * h)
            assert abs(num - grad[idx]) < 1e-6, (name, idx, num, grad[idx])


def torch_sdpa_grads(q, k, v, do, scale, attn_mask=None):
    tq, tk, tv = (torch.from_numpy(x).clone().requires_grad_() for x in (q, k, v))
    o = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=attn_mask,
                                                         scale=scale)
    o.backward(torch.from_numpy(do))
    return tq.grad.numpy(), tk.grad.numpy(), tv.grad.numpy()


def test_backward_dense_matches_torch_autograd():
    n, D = 300, 16
    q, k, v, do = (rand((2, n, D), s) for s in (55, 56, 57, 58))
    rp, ci = ro.full_csr(n, 128)
    got = ro.attention_backward(q, k, v, do, rp, ci, scale=0.3)
    ref = torch_sdpa_grads(q, k, v, do, 0.3)
    for a, b in zip(got, ref):
        assert np.abs(a - b).max() < 1e-11


def test_backward_element_single_frame_matches_torch_band():
    n, w0, D = 400, 30, 8
    q, k, v, do = (rand((n, D), s) for s in (59, 60, 61, 62))
    rp, ci = ro.csr(ro.block_mask(1, n, w0))
    got = ro.attention_backward(q, k, v, do, rp, ci, scale=0.5, element=(n, w0))
    i = np.arange(n)
    band = torch.from_numpy(np.abs(i[:, None] - i[None, :]) < w0)
    ref = torch_sdpa_grads(q[None], k[None], v[None], do[None], 0.5, attn_mask=band)
    for a, b in zip(got, ref):
        assert np.abs(a - b[0]).max() < 1e-11


def test_backward_closed_forms():
    """Rows of P sum to one, so sum_j dv_j = sum_i do_i; scale 0 gives dq = dk = 0."""
    F, S, w0 = 4, 200, 20
    n = F * S
    q, k, v, do = (rand((n, 8), s) for s in (63, 64, 65, 66))
    rp, ci = ro.csr(ro.block_mask(F, S, w0))
    dq, dk, dv = ro.attention_backward(q, k, v, do, rp, ci, scale=0.25)
    assert np.abs(dv.sum(axis=0) - do.sum(axis=0)).max() < 1e-10
    dq0, dk0, dv0 = ro.attention_backward(q, k, v, do, rp, ci, scale=0.0)
    assert np.abs(dq0).max() == 0 and np.abs(dk0).max() == 0
    assert np.abs(dv0.sum(axis=0) - do.sum(axis=0)).max() < 1e-10


def test_transpose_csr_vs_dense():
    F, S, w0 = 5, 300, 40
    bm = ro.block_mask(F, S, w0)
    rp, ci = ro.csr(bm)
    cp, ri = ro.transpose_csr(rp, ci, bm.shape[0])
    rp_t, ci_t = ro.csr(bm.T.copy())
    assert np.array_equal(cp, rp_t) and np.array_equal(ri, ci_t)
    # A non-symmetric mask too.
    rng = np.random.default_rng(5)
    m = rng.random((23, 23)) < 0.3
    rp, ci = ro.csr(m)
    cp, ri = ro.transpose_csr(rp, ci, 23)
    rp_t, ci_t = ro.csr(m.T.copy())
    assert np.array_equal(cp, rp_t) and np.array_equal(ri, ci_t)


def test_backward_restriction_matches_full():
    F, S, w0 = 5, 300, 40
    n = F * S
    q, k, v, do = (rand((n, 8), s) for s in (67, 68, 69, 70))
    rp, ci = ro.csr(ro.block_mask(F, S, w0))
    full = ro.attention_backward(q, k, v, do, rp, ci, scale=0.4)
    part = ro.attention_backward(q, k, v, do, rp, ci, scale=0.4, query_blocks=[1, 5],
                                 key_blocks=[0, 7, 11])
    rows_q = np.r_[128:256, 640:768]
    rows_k = np.r_[0:128, 896:1024, 1408:n]
    assert np.array_equal(part[0][rows_q], full[0][rows_q])
    for a, b in zip(part[1:], full[1:]):
        assert np.array_equal(a[rows_k], b[rows_k])
    assert np.isnan(part[0][0]).all() and np.isnan(part[1][200]).all()
