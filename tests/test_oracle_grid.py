"""Pins for the oracle's 2-D grid variant (a frame as an H x W latent grid, Manhattan
spatial distance), each checked against something other than the oracle itself.

* Brute force. Pure-Python loops: grid positions enumerated row by row (no division),
  the window taken as the exact rational W0 / 2**floor(math.log2(d + 1)).
* Closed forms. The lattice points within Manhattan distance r of an interior point
  number 2r^2 + 2r + 1.
* Special cases. A grid of one row, or of one column, is the 1-D rule; a transposed
  grid gives the same mask after the matching permutation of tokens.
* Library routines. torch's scaled_dot_product_attention in fp64 with a boolean mask
  built by the brute-force loops.
"""
import math
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import radial_oracle as ro


def grid_positions(H, W):
    """(row, col) of each in-frame index, listed in storage order (row by row)."""
    pos = []
    for y in range(H):
        for x in range(W):
            pos.append((y, x))
    return pos


def bf_allowed_grid(t_q, t_k, H, W, w0, pos):
    S = H * W
    fq, sq = divmod(t_q, S)
    fk, sk = divmod(t_k, S)
    (yq, xq), (yk, xk) = pos[sq], pos[sk]
    window = Fraction(w0, 2 ** math.floor(math.log2(abs(fq - fk) + 1)))
    return abs(yq - yk) + abs(xq - xk) < window


def bf_element_mask_grid(F, H, W, w0):
    pos = grid_positions(H, W)
    n = F * H * W
    return np.array([[bf_allowed_grid(i, j, H, W, w0, pos) for j in range(n)]
                     for i in range(n)])


SHAPES = [  # (F, H, W, W0)
    (1, 5, 7, 4), (2, 4, 6, 1), (3, 3, 5, 7), (4, 6, 4, 9), (5, 2, 9, 3),
    (3, 7, 3, 12), (6, 3, 3, 5), (2, 8, 8, 15),
]


@pytest.mark.parametrize("F,H,W,w0", SHAPES)
def test_grid_mask_vs_exact_rational_bruteforce(F, H, W, w0):
    assert np.array_equal(ro.element_mask(F, H * W, w0, grid_w=W),
                          bf_element_mask_grid(F, H, W, w0))


def test_grid_edge_windows():
    # The largest distance is (H - 1) + (W - 1); W0 around it, and around it times 2^k.
    F, H, W = 5, 4, 6
    top = H + W - 2
    for w0 in (1, top, top + 1, 2 * top, 2 * top + 1, 4 * top, 4 * top + 1):
        assert np.array_equal(ro.element_mask(F, H * W, w0, grid_w=W),
                              bf_element_mask_grid(F, H, W, w0)), w0


def test_one_row_or_one_column_is_the_1d_rule():
    # One row: the column index is s itself. One column: the row index is s itself.
    for F, S, w0 in [(4, 30, 7), (3, 50, 60), (6, 12, 5)]:
        one_d = ro.element_mask(F, S, w0)
        assert np.array_equal(ro.element_mask(F, S, w0, grid_w=S), one_d)
        assert np.array_equal(ro.element_mask(F, S, w0, grid_w=1), one_d)
        assert np.array_equal(ro.block_mask(F, S, w0, block=8, grid_w=S),
                              ro.block_mask(F, S, w0, block=8))


def test_diamond_count_closed_form():
    """An interior query sees 2r^2 + 2r + 1 keys of a frame at radius r."""
    H = W = 31
    S = H * W
    centre = 15 * W + 15
    for r in range(0, 16):
        m = ro.element_mask(1, S, r + 1, grid_w=W)
        assert m[centre].sum() == 2 * r * r + 2 * r + 1, r
    # Frame distance 2 (band 1): radius (W0 - 1) >> 1 in the other frame.
    w0 = 20
    r = (w0 - 1) >> 1
    m = ro.element_mask(3, S, w0, grid_w=W)
    assert m[centre, 2 * S:].sum() == 2 * r * r + 2 * r + 1
    # Frame distance 7 (band 3): radius (W0 - 1) >> 3.
    m = ro.element_mask(8, S, 50, grid_w=W)
    r = 49 >> 3
    assert m[centre, 7 * S:].sum() == 2 * r * r + 2 * r + 1


def test_transposed_grid_is_a_permutation():
    """Row and column play the same part: the H x W mask equals the W x H mask after
    renumbering each token (y, x) as (x, y)."""
    F, H, W, w0 = 3, 4, 7, 6
    S = H * W
    perm = np.array([f * S + x * H + y for f in range(F) for y in range(H) for x in range(W)])
    a = ro.element_mask(F, S, w0, grid_w=W)
    b = ro.element_mask(F, S, w0, grid_w=H)
    assert np.array_equal(a, b[np.ix_(perm, perm)])
    assert not np.array_equal(a, b)  # the renumbering is needed


@pytest.mark.parametrize("F,H,W,w0", [(5, 6, 8, 9), (3, 10, 13, 7), (8, 4, 5, 6)])
def test_grid_invariants(F, H, W, w0):
    S = H * W
    m = ro.element_mask(F, S, w0, grid_w=W)
    assert m.diagonal().all()
    assert np.array_equal(m, m.T)
    blocks = m.reshape(F, S, F, S)
    for c in range(1, F):
        assert np.array_equal(blocks[c:, :, c:, :], blocks[:-c, :, :-c, :])
    assert (ro.element_mask(F, S, w0 + 1, grid_w=W) | ~m).all()


@pytest.mark.parametrize("F,H,W,w0,block", [
    (4, 6, 9, 7, 16), (3, 10, 13, 11, 32), (7, 5, 5, 4, 8), (2, 12, 20, 25, 128),
    (5, 9, 11, 3, 128), (3, 30, 52, 81, 128),
])
def test_grid_block_counts_vs_element_reduction(F, H, W, w0, block):
    counts = ro.block_counts(F, H * W, w0, block, grid_w=W)
    ref = ro.block_counts_from_elements(ro.element_mask(F, H * W, w0, grid_w=W), block)
    assert np.array_equal(counts, ref)


def test_grid_width_must_divide_the_frame():
    with pytest.raises(ValueError):
        ro.element_mask(2, 30, 5, grid_w=7)
    with pytest.raises(ValueError):
        ro.block_mask(2, 30, 5, grid_w=0)


def test_grid_element_attention_vs_torch_sdpa():
    """Element semantics on the grid: torch's fp64 attention with the brute-force mask."""
    F, H, W, w0, D = 3, 9, 14, 8, 16
    S = H * W
    n = F * S
    rng = np.random.default_rng(51)
    q, k, v = (rng.standard_normal((2, n, D)) for _ in range(3))
    rp, ci = ro.csr(ro.block_mask(F, S, w0, grid_w=W))
    o, _ = ro.attention(q, k, v, rp, ci, scale=0.35, element=(S, w0, W))
    bm = torch.from_numpy(bf_element_mask_grid(F, H, W, w0))
    ref = torch.nn.functional.scaled_dot_product_attention(
        *(torch.from_numpy(x) for x in (q, k, v)), attn_mask=bm, scale=0.35).numpy()
    assert np.abs(o - ref).max() < 1e-12


def test_grid_element_backward_vs_torch_autograd():
    F, H, W, w0, D = 3, 6, 11, 6, 8
    S = H * W
    n = F * S
    rng = np.random.default_rng(52)
    q, k, v, do = (rng.standard_normal((n, D)) for _ in range(4))
    rp, ci = ro.csr(ro.block_mask(F, S, w0, grid_w=W))
    got = ro.attention_backward(q, k, v, do, rp, ci, 0.5, element=(S, w0, W))
    bm = torch.from_numpy(bf_element_mask_grid(F, H, W, w0))
    qt, kt, vt = (torch.from_numpy(x).requires_grad_() for x in (q, k, v))
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=bm, scale=0.5)
    o.backward(torch.from_numpy(do))
    for g, t in zip(got, (qt, kt, vt)):
        assert np.abs(g - t.grad.numpy()).max() < 1e-10
