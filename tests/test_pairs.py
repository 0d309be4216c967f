"""The pair table (radial_build_pairs): which query-block rows the kernel computes together.

A pairing changes no result, only which rows share a workgroup, so these tests check
that a table is a valid schedule (every row exactly once, a < b in a pair, the pairs
ordered by union-length band and then by first row), that it is
deterministic, and that on the radial masks it never makes the shared walk longer than
the adjacent pairing (2p, 2p + 1). GPU tests check that the output does not depend on
the table.
"""
import ctypes
import time

import numpy as np
import pytest
import torch

import block_sparse_attention_radial_amd as radial
from block_sparse_attention_radial_amd.inputs import WORKLOADS

INVALID = -1


def union_walk(rows, table):
    """Tiles the kernel walks: the union of each pair's two key-block sets."""
    return sum(len(rows[a] | (rows[b] if b >= 0 else set())) for a, b in table)


def row_sets(mask):
    rp, ci = mask.row_ptr.numpy(), mask.col_idx.numpy()
    return [set(ci[rp[i]:rp[i + 1]].tolist()) for i in range(mask.nb)]


def union_length(rows, a, b):
    return len(rows[a] | (rows[b] if b >= 0 else set()))


def check_partition(table, nb, rows=None):
    t = np.asarray(table).reshape(-1, 2)
    assert (nb + 1) // 2 <= len(t) <= nb
    firsts = t[:, 0]
    if rows is not None:  # bands of 16 blocks of union length, longest first; then by row
        key = [(-(union_length(rows, a, b) // 16), a) for a, b in t]
        assert key == sorted(key), "pairs ordered by union-length band, then first row"
    seconds = t[:, 1]
    assert np.all((seconds == -1) | (seconds > firsts)), "a < b or a single row"
    listed = np.concatenate([firsts, seconds[seconds >= 0]])
    assert np.array_equal(np.sort(listed), np.arange(nb)), "every row exactly once"


@pytest.mark.parametrize("key", list(WORKLOADS))
def test_workload_tables_are_valid_and_never_longer_than_adjacent(key):
    wl = WORKLOADS[key]
    m = radial.build_mask(wl.frames, wl.tokens_per_frame, wl.w0)
    table = m.pairs.numpy()
    rows = row_sets(m)
    check_partition(table, m.nb, rows)
    adjacent = [(2 * p, 2 * p + 1 if 2 * p + 1 < m.nb else -1) for p in range((m.nb + 1) // 2)]
    assert union_walk(rows, table) <= union_walk(rows, adjacent)
    # Radial masks leave no row alone except the odd one out.
    assert len(table) == (m.nb + 1) // 2


def test_long_video_table_shortens_the_walk():
    """At 4x length the frame-distance partners cut the walk by more than 10%."""
    wl = WORKLOADS["long4x"]
    m = radial.build_mask(wl.frames, wl.tokens_per_frame, wl.w0)
    rows = row_sets(m)
    adjacent = [(2 * p, 2 * p + 1) for p in range(m.nb // 2)]
    assert union_walk(rows, m.pairs.numpy()) < 0.9 * union_walk(rows, adjacent)


def test_deterministic():
    wl = WORKLOADS["hunyuan"]
    m = radial.build_mask(wl.frames, wl.tokens_per_frame, wl.w0)
    again = radial.build_pairs(m.row_ptr, m.col_idx, wl.tokens_per_frame)
    assert torch.equal(m.pairs, again)


def test_build_mask_without_pairs():
    assert radial.build_mask(4, 256, 256, pairs=False).pairs is None


@pytest.mark.parametrize("nb", [1, 2, 3, 5, 8, 37])
def test_small_and_odd_sizes(nb):
    rng = np.random.default_rng(nb)
    rows = [np.flatnonzero(rng.random(nb) < 0.4).astype(np.int32) for _ in range(nb)]
    rp = np.zeros(nb + 1, np.int32)
    rp[1:] = np.cumsum([len(r) for r in rows])
    ci = np.concatenate(rows + [np.zeros(0, np.int32)])
    for tpf in (0, 256, 1000):
        table = radial.build_pairs(torch.from_numpy(rp), torch.from_numpy(ci), tpf).numpy()
        check_partition(table, nb, [set(r.tolist()) for r in rows])
        assert len(table) == (nb + 1) // 2


def test_dense_rows_pair_with_their_neighbour():
    """All rows equal: every candidate scores the same, and ties go to offset 1."""
    m = radial.dense_mask(40 * 128)
    table = radial.build_pairs(m.row_ptr, m.col_idx, 1280).numpy()
    assert table.tolist() == [[2 * p, 2 * p + 1] for p in range(20)]


def test_unsorted_rows_still_give_a_valid_schedule():
    rng = np.random.default_rng(3)
    nb = 50
    rows = [rng.permutation(nb)[: rng.integers(1, nb)].astype(np.int32) for _ in range(nb)]
    rp = np.zeros(nb + 1, np.int32)
    rp[1:] = np.cumsum([len(r) for r in rows])
    table = radial.build_pairs(torch.from_numpy(rp), torch.from_numpy(np.concatenate(rows)), 0)
    check_partition(table.numpy(), nb)


def test_large_dense_mask_is_cheap():
    """Past the work bound the builder returns the adjacent pairing without scoring."""
    nb = 3900
    m = radial.dense_mask(nb * 128)
    t0 = time.perf_counter()
    table = radial.build_pairs(m.row_ptr, m.col_idx, 1280).numpy()
    assert time.perf_counter() - t0 < 5.0
    assert table.tolist() == [[2 * p, 2 * p + 1] for p in range(nb // 2)]


def test_errors():
    lib = radial.lib()
    rp = (ctypes.c_int32 * 3)(0, 1, 2)
    ci = (ctypes.c_int32 * 2)(0, 1)
    out = (ctypes.c_int32 * 4)()
    npairs = ctypes.c_int32()
    ok = lib.radial_build_pairs(2, rp, ci, 0, out, ctypes.byref(npairs))
    assert ok == 0 and npairs.value == 1 and list(out)[:2] == [0, 1]
    assert lib.radial_build_pairs(0, rp, ci, 0, out, ctypes.byref(npairs)) == INVALID
    assert lib.radial_build_pairs(2, rp, ci, -1, out, ctypes.byref(npairs)) == INVALID
    assert lib.radial_build_pairs(2, None, ci, 0, out, ctypes.byref(npairs)) == INVALID
    assert lib.radial_build_pairs(2, rp, None, 0, out, ctypes.byref(npairs)) == INVALID
    assert lib.radial_build_pairs(2, rp, ci, 0, None, ctypes.byref(npairs)) == INVALID
    assert lib.radial_build_pairs(2, rp, ci, 0, out, None) == INVALID
    bad_start = (ctypes.c_int32 * 3)(1, 1, 2)
    assert lib.radial_build_pairs(2, bad_start, ci, 0, out, ctypes.byref(npairs)) == INVALID
    decreasing = (ctypes.c_int32 * 3)(0, 2, 1)
    assert lib.radial_build_pairs(2, decreasing, ci, 0, out, ctypes.byref(npairs)) == INVALID
