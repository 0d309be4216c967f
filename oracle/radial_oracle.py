"""Plain CPU oracle for the Radial Attention forward pass (numpy, fp64).

TEST INFRASTRUCTURE ONLY. The tests, the smoke check and the benchmark's CPU-baseline leg
are the only code that may import or run this module. The library never does, and this
module imports nothing from the library.

What it computes follows these pages:

* "Radial Attention: O(n log n) Sparse Attention with Energy Decay for Long Video
  Generation" (paper summary page), Outline. Attention goes only to spatially close
  tokens, and the window gets smaller as the temporal distance grows.
* "Radial Attention: A Breakthrough in Efficient Long Video Generation", How Radial
  Attention Works. The mask is static. Compute density halves each time the temporal
  distance doubles. The mask is applied in 128x128 blocks.
* The radial-attention-video SKILL.md page. Step 1 gives the frame-major token
  coordinates (frame = t // S, spatial = t % S) and masked positions as -inf before the
  softmax. Step 2 gives scores = Q K^T * head_dim**-0.5, then softmax, then times V, with
  one mask broadcast over every batch and head.

The pages leave some steps open. This module takes the plainest reading of each:

1. The spatial window at temporal distance d = |f_q - f_k| is W0 / 2**floor(log2(d + 1)),
   so it halves every time d + 1 doubles. The test is exact and strict:
   allowed(q, k) <=> |s_q - s_k| * 2**floor(log2(d + 1)) < W0.
2. Spatial distance is the 1-D distance between in-frame token indices.
3. Block semantics. A block pair is active iff at least one element in it is allowed.
   Every real key of an active block takes part in the softmax. Keys at or past the
   sequence end never take part.
4. Element semantics (an option of `attention`): the rule of reading 1 also removes the
   single disallowed entries inside the active blocks, as -inf scores before the
   softmax. The diagonal is always allowed (W0 >= 1), so no row is left empty.
5. The backward pass (`attention_backward`) is the vector-Jacobian product of the
   same softmax attention over the same key sets; the pages use it for LoRA
   fine-tuning (the SKILL.md page, Step 4: loss.backward() through the attention).
6. The 2-D grid variant (the SKILL.md page, Step 1, its grid-distance helper): a frame is
   a latent grid of H rows and W columns stored row by row (S = H * W), so spatial index
   s sits at row s // W and column s % W, and the spatial distance is the Manhattan
   distance |row_q - row_k| + |col_q - col_k|. The helper takes a square grid of side
   sqrt(S); here the caller gives W, and H = S / W. Everything else stays as in reading
   1: allowed(q, k) <=> distance * 2**floor(log2(d + 1)) < W0. W = S (one row) is the
   1-D rule of reading 2. The page's other helper, which folds the temporal distance
   into one combined distance with constants lost from the text, is not used.

Parity pins for every function here are in tests/test_oracle.py. Each pin checks the
function against something other than itself: brute force with exact rationals, closed
forms, invariants, or library routines.
"""
from __future__ import annotations

import numpy as np

BLOCK = 128


# --------------------------------------------------------------------------------------
# Mask rule (element level)
# --------------------------------------------------------------------------------------

def band(d):
    """floor(log2(d + 1)) for integer d >= 0, computed exactly.

    For an integer x >= 1, frexp gives x = m * 2**e with 0.5 <= m < 1, so floor(log2 x)
    is e - 1. There is no rounding because integers below 2**53 are exact in a double.
    """
    d = np.asarray(d, dtype=np.int64)
    return (np.frexp((d + 1).astype(np.float64))[1] - 1).astype(np.int64)


def token_coords(frames: int, tokens_per_frame: int):
    """Frame-major flattening: token t sits in frame t // S at spatial index t % S."""
    t = np.arange(frames * tokens_per_frame, dtype=np.int64)
    return t // tokens_per_frame, t % tokens_per_frame


def spatial_distance(sq, sk, grid_w=None):
    """In-frame distance: |s_q - s_k| (reading 2), or with a grid width W the Manhattan
    distance between (s // W, s % W) positions (reading 6)."""
    sq, sk = np.asarray(sq, dtype=np.int64), np.asarray(sk, dtype=np.int64)
    if grid_w is None:
        return np.abs(sq - sk)
    return np.abs(sq // grid_w - sk // grid_w) + np.abs(sq % grid_w - sk % grid_w)


def check_grid(tokens_per_frame: int, grid_w):
    if grid_w is not None and (grid_w < 1 or tokens_per_frame % grid_w):
        raise ValueError("the grid width must divide the tokens per frame")


def allowed(fq, sq, fk, sk, w0, grid_w=None):
    """Element rule: distance(s_q, s_k) * 2**floor(log2(|f_q - f_k| + 1)) < W0 (reading 1;
    the distance of reading 2, or of reading 6 with a grid width)."""
    fq, fk = np.asarray(fq, dtype=np.int64), np.asarray(fk, dtype=np.int64)
    return spatial_distance(sq, sk, grid_w) * (np.int64(1) << band(np.abs(fq - fk))) < w0


def element_mask(frames: int, tokens_per_frame: int, w0: int, grid_w=None) -> np.ndarray:
    """The n x n boolean mask with the rule applied to every (query, key) pair.

    Only for small n, because it materialises n**2 booleans.
    """
    check_grid(tokens_per_frame, grid_w)
    f, s = token_coords(frames, tokens_per_frame)
    return allowed(f[:, None], s[:, None], f[None, :], s[None, :], w0, grid_w)


# --------------------------------------------------------------------------------------
# Block reduction (128 x 128 blocks)
# --------------------------------------------------------------------------------------

def num_blocks(n: int, block: int = BLOCK) -> int:
    return (n + block - 1) // block


def block_counts_from_elements(mask: np.ndarray, block: int = BLOCK) -> np.ndarray:
    """Allowed-element count per (query block, key block), from an explicit element mask.

    The sequence is padded with disallowed entries up to a whole number of blocks, so
    padding never counts.
    """
    n = mask.shape[0]
    nb = num_blocks(n, block)
    padded = np.zeros((nb * block, nb * block), dtype=np.int64)
    padded[:n, :n] = mask
    return padded.reshape(nb, block, nb, block).sum(axis=(1, 3))


def _frame_pieces(n: int, tokens_per_frame: int, block: int):
    """Split each block's token range where a frame starts.

    Returns an int64 array of rows (block, frame, s_begin, s_end) with s_end exclusive.
    The pieces of one block tile its real tokens exactly.
    """
    rows = []
    for b in range(num_blocks(n, block)):
        t, t_end = b * block, min(n, (b + 1) * block)
        while t < t_end:
            f = t // tokens_per_frame
            stop = min(t_end, (f + 1) * tokens_per_frame)
            rows.append((b, f, t - f * tokens_per_frame, stop - f * tokens_per_frame))
            t = stop
    return np.asarray(rows, dtype=np.int64).reshape(-1, 4)


def block_counts(frames: int, tokens_per_frame: int, w0: int,
                 block: int = BLOCK, grid_w=None) -> np.ndarray:
    """Allowed-element count per (query block, key block), for any size.

    The rule depends only on the band of |f_q - f_k| and on (s_q, s_k). So for each band
    value that occurs, the S x S in-frame mask is tabulated and turned into a
    summed-area table with cumsum. An element count over any rectangle of that mask
    then costs four lookups. A block pair is a union of rectangles, one per (query
    frame piece, key frame piece). The count is an exact integer. `grid_w` selects the
    2-D grid distance (reading 6).
    """
    check_grid(tokens_per_frame, grid_w)
    S = tokens_per_frame
    n = frames * S
    nb = num_blocks(n, block)
    s = np.arange(S, dtype=np.int64)
    max_band = int(band(frames - 1))
    sat = np.zeros((max_band + 1, S + 1, S + 1), dtype=np.int64)
    for kk in range(max_band + 1):
        inframe = spatial_distance(s[:, None], s[None, :], grid_w) * (np.int64(1) << kk) < w0
        sat[kk, 1:, 1:] = inframe.astype(np.int64).cumsum(axis=0).cumsum(axis=1)

    pieces = _frame_pieces(n, S, block)
    kb, kf, k0, k1 = pieces.T
    counts = np.zeros((nb, nb), dtype=np.int64)
    for qb, qf, q0, q1 in pieces:
        bb = band(np.abs(qf - kf))
        rect = sat[bb, q1, k1] - sat[bb, q0, k1] - sat[bb, q1, k0] + sat[bb, q0, k0]
        np.add.at(counts[qb], kb, rect)
    return counts


def block_mask(frames: int, tokens_per_frame: int, w0: int,
               block: int = BLOCK, grid_w=None) -> np.ndarray:
    """Block (a, b) is active iff it holds at least one allowed element (reading 3)."""
    return block_counts(frames, tokens_per_frame, w0, block, grid_w) > 0


def csr(bmask: np.ndarray):
    """Compressed rows of a block mask: row_ptr[nb + 1] and ascending col_idx (int32).

    This form is unique for a given mask, so two CSRs agree bit for bit iff the masks do.
    """
    bmask = np.asarray(bmask, dtype=bool)
    row_ptr = np.zeros(bmask.shape[0] + 1, dtype=np.int64)
    row_ptr[1:] = np.cumsum(bmask.sum(axis=1))
    col_idx = np.nonzero(bmask)[1]
    return row_ptr.astype(np.int32), col_idx.astype(np.int32)


def row_keys(row_ptr, col_idx, qb: int, n: int, block: int = BLOCK) -> np.ndarray:
    """Key token indices that query block qb attends: every real key of its blocks."""
    cols = col_idx[row_ptr[qb]:row_ptr[qb + 1]]
    if len(cols) == 0:
        return np.zeros(0, dtype=np.int64)
    keys = (np.asarray(cols, dtype=np.int64)[:, None] * block
            + np.arange(block, dtype=np.int64)[None, :]).reshape(-1)
    return keys[keys < n]


# --------------------------------------------------------------------------------------
# Attention over the active key set
# --------------------------------------------------------------------------------------

def element_allowed(element, rows: slice, keys) -> np.ndarray:
    """The element rule between the query rows `rows` and the key tokens `keys`;
    element = (tokens_per_frame, w0) or (tokens_per_frame, w0, grid_w)."""
    S, w0, *grid = element
    grid_w = grid[0] if grid else None
    check_grid(S, grid_w)
    qi = np.arange(rows.start, rows.stop, dtype=np.int64)[:, None]
    kj = np.asarray(keys, dtype=np.int64)[None, :]
    return allowed(qi // S, qi % S, kj // S, kj % S, w0, grid_w)


def attention(q, k, v, row_ptr, col_idx, scale: float, block: int = BLOCK,
              query_blocks=None, element=None):
    """fp64 softmax attention, each query block over the keys of its active blocks.

    q, k, v have shape [..., n, D]; leading dims (batch, heads) share one mask. For query
    row i with key set K_i: x_j = scale * <q_i, k_j>, p_j = exp(x_j - max x), and
    o_i = sum_j p_j v_j / sum_j p_j. Subtracting the max only avoids overflow; the result
    is the same softmax. Returns (o, lse) with lse_i = max x + ln(sum_j p_j), i.e. the
    natural-log log-sum-exp of the scaled scores. Rows of query blocks not listed in
    `query_blocks` are left as NaN.

    element = (tokens_per_frame, w0) switches to element semantics: inside K_i, only the
    keys j that the element rule allows for (i, j) take part (the SKILL.md page, Step 1:
    masked positions are -inf before the softmax). The block mask stays the set of
    blocks visited; the rule removes single entries inside them. A third entry,
    (tokens_per_frame, w0, grid_w), takes the 2-D grid distance (reading 6).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    n = q.shape[-2]
    nb = num_blocks(n, block)
    o = np.full(q.shape[:-1] + (v.shape[-1],), np.nan)
    lse = np.full(q.shape[:-1], np.nan)
    for qb in (range(nb) if query_blocks is None else query_blocks):
        rows = slice(qb * block, min(n, (qb + 1) * block))
        keys = row_keys(row_ptr, col_idx, qb, n, block)
        x = scale * (q[..., rows, :] @ np.swapaxes(k[..., keys, :], -1, -2))
        if element is not None:
            x = np.where(element_allowed(element, rows, keys), x, -np.inf)
        m = x.max(axis=-1, keepdims=True)
        p = np.exp(x - m)
        denom = p.sum(axis=-1, keepdims=True)
        o[..., rows, :] = (p @ v[..., keys, :]) / denom
        lse[..., rows] = (m + np.log(denom))[..., 0]
    return o, lse


def attention_backward(q, k, v, do, row_ptr, col_idx, scale: float, block: int = BLOCK,
                       element=None, query_blocks=None, key_blocks=None):
    """fp64 gradients (dq, dk, dv) of `attention` for the output cotangent do.

    This is the vector-Jacobian product of softmax attention over the same key sets
    (the radial-attention-video SKILL.md page, Step 4, fine-tunes through the attention
    with loss.backward()). Per query row i with key set K_i, P = softmax(scale q K^T)
    over K_i and o_i = P V:
        dv_j += P_ij do_i,    dP_ij = <do_i, v_j>,    dS_ij = P_ij (dP_ij - <do_i, o_i>),
        dq_i = scale sum_j dS_ij k_j,    dk_j += scale dS_ij q_i.
    The identity sum_j P_ij dP_ij = <do_i, o_i> is what makes dS the softmax Jacobian
    applied to dP. `element` is as in `attention`.

    `query_blocks` / `key_blocks` (optional) restrict the work to the dq rows of those
    query blocks and the dk, dv rows of those key blocks (the rest is left NaN): only the
    query blocks listed, and those whose rows hold one of the key blocks, are processed.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    n = q.shape[-2]
    nb = num_blocks(n, block)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    todo = range(nb)
    if query_blocks is not None or key_blocks is not None:
        qs = set(query_blocks or [])
        ks = set(key_blocks or [])
        todo = [qb for qb in range(nb) if qb in qs
                or ks.intersection(np.asarray(col_idx[row_ptr[qb]:row_ptr[qb + 1]]).tolist())]
    for qb in todo:
        rows = slice(qb * block, min(n, (qb + 1) * block))
        keys = row_keys(row_ptr, col_idx, qb, n, block)
        x = scale * (q[..., rows, :] @ np.swapaxes(k[..., keys, :], -1, -2))
        if element is not None:
            x = np.where(element_allowed(element, rows, keys), x, -np.inf)
        p = np.exp(x - x.max(axis=-1, keepdims=True))
        p /= p.sum(axis=-1, keepdims=True)
        o = p @ v[..., keys, :]
        g = do[..., rows, :]
        dp = g @ np.swapaxes(v[..., keys, :], -1, -2)
        ds = p * (dp - (g * o).sum(axis=-1, keepdims=True))
        dq[..., rows, :] = scale * (ds @ k[..., keys, :])
        dk[..., keys, :] += scale * (np.swapaxes(ds, -1, -2) @ q[..., rows, :])
        dv[..., keys, :] += np.swapaxes(p, -1, -2) @ g
    if query_blocks is not None or key_blocks is not None:
        keep_q = np.zeros(n, dtype=bool)
        keep_k = np.zeros(n, dtype=bool)
        for qb in query_blocks or []:
            keep_q[qb * block:(qb + 1) * block] = True
        for kb in key_blocks or []:
            keep_k[kb * block:(kb + 1) * block] = True
        dq[..., ~keep_q, :] = np.nan
        dk[..., ~keep_k, :] = np.nan
        dv[..., ~keep_k, :] = np.nan
    return dq, dk, dv


def transpose_csr(row_ptr, col_idx, nb: int):
    """Column-major view of a block mask: for key block c, the query blocks whose rows
    list it, ascending (the CSR of the transposed mask)."""
    rows = np.repeat(np.arange(nb, dtype=np.int64), np.diff(np.asarray(row_ptr)))
    cols = np.asarray(col_idx, dtype=np.int64)
    order = np.lexsort((rows, cols))
    col_ptr = np.zeros(nb + 1, dtype=np.int32)
    np.add.at(col_ptr, cols + 1, 1)
    return np.cumsum(col_ptr).astype(np.int32), rows[order].astype(np.int32)


def full_csr(n: int, block: int = BLOCK):
    """The CSR of the all-active block mask (every query block sees every key block)."""
    return csr(np.ones((num_blocks(n, block),) * 2, dtype=bool))

