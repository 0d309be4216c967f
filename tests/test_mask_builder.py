"""The library's host mask builder against the CPU oracle, bit for bit.

The builder sweeps closed-form key intervals per frame piece. The oracle counts allowed
elements with summed-area tables. The two share no code, so agreement on every shape
is a real check.
"""
import hashlib
import json
import os

import numpy as np
import pytest

import block_sparse_attention_radial_amd as radial
from block_sparse_attention_radial_amd.inputs import WORKLOADS
from oracle import radial_oracle as ro

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "masks.json")


def lib_csr(F, S, w0):
    m = radial.build_mask(F, S, w0)
    return m.row_ptr.numpy(), m.col_idx.numpy()


def oracle_csr(F, S, w0):
    return ro.csr(ro.block_mask(F, S, w0))


def assert_same(F, S, w0):
    rp, ci = lib_csr(F, S, w0)
    orp, oci = oracle_csr(F, S, w0)
    assert rp.dtype == np.int32 and ci.dtype == np.int32
    assert np.array_equal(rp, orp), (F, S, w0)
    assert np.array_equal(ci, oci), (F, S, w0)


@pytest.mark.parametrize("key", ["tiny", "small", "wan"])
def test_workloads_bit_exact(key):
    wl = WORKLOADS[key]
    assert_same(wl.frames, wl.tokens_per_frame, wl.w0)


@pytest.mark.slow
@pytest.mark.parametrize("key", ["hunyuan", "long4x"])
def test_large_workloads_bit_exact(key):
    wl = WORKLOADS[key]
    assert_same(wl.frames, wl.tokens_per_frame, wl.w0)


@pytest.mark.parametrize("F,S,w0", [
    (6, 1000, 100),    # 34% dense, ragged last block of 112 rows
    (8, 1000, 334),    # ragged, about half dense
    (12, 100, 37),     # frames shorter than a block
    (1, 5000, 1),      # one frame, window 1: only the diagonal blocks
    (1, 129, 1),       # two blocks, the second holds one token
    (3, 1, 1),         # one token per frame, three tokens in all
    (5, 333, 10**6),   # huge window: block-dense
    (40, 64, 2),       # many short frames
    (21, 1560, 1559),  # one below the Wan window
    (21, 1560, 1561),
])
def test_edge_shapes_bit_exact(F, S, w0):
    assert_same(F, S, w0)


def test_random_sweep_bit_exact():
    rng = np.random.default_rng(0)
    for _ in range(40):
        F = int(rng.integers(1, 17))
        S = int(rng.integers(1, 1601))
        w0 = int(rng.integers(1, 2 * S + 2))
        assert_same(F, S, w0)


def test_golden_digests():
    with open(GOLDEN) as f:
        gold = json.load(f)
    for case in gold["cases"]:
        rp, ci = lib_csr(case["frames"], case["tokens_per_frame"], case["w0"])
        h = hashlib.sha256()
        h.update(rp.astype("<i4").tobytes())
        h.update(ci.astype("<i4").tobytes())
        assert h.hexdigest() == case["sha256"], case["name"]
        assert len(rp) - 1 == case["nb"] and len(ci) == case["nnz"]


def test_mask_dims_agree_with_build():
    for F, S, w0 in [(21, 1560, 1560), (6, 1000, 100), (1, 1, 1)]:
        nb, nnz = radial.mask_dims(F, S, w0)
        m = radial.build_mask(F, S, w0)
        assert (nb, nnz) == (m.nb, m.nnz)


def test_dense_mask_helper():
    m = radial.dense_mask(1000)
    rp, ci = ro.full_csr(1000)
    assert np.array_equal(m.row_ptr.numpy(), rp) and np.array_equal(m.col_idx.numpy(), ci)
