"""C-ABI checks that need no GPU: exported symbols, error codes, argument validation.

radial_attn_fwd validates everything on the host before its first HIP call, so every
error path is reachable here with fake (never dereferenced) pointer values.
"""
import ctypes
import os
import re
import subprocess

import pytest

import block_sparse_attention_radial_amd as radial
from block_sparse_attention_radial_amd import api

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "radial_attn.h")

OK, INVALID, HEADDIM, CAPACITY, SHAPE, MISALIGNED, TOO_LARGE, HIP = 0, -1, -2, -3, -4, -5, -6, -7


def declared_symbols():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(radial_\w+)\s*\(", text, re.M)))


def test_header_declares_the_boundary():
    assert declared_symbols() == sorted(
        ["radial_mask_dims", "radial_build_mask", "radial_mask_dims_grid",
         "radial_build_mask_grid", "radial_build_pairs", "radial_attn_fwd", "radial_attn_fwd_rule",
         "radial_attn_fwd_varlen", "radial_transpose_mask", "radial_attn_bwd",
         "radial_attn_bwd_varlen", "radial_attn_fwd_varlen_rule", "radial_attn_bwd_noalloc",
         "radial_element_table_bytes", "radial_build_element_table",
         "radial_attn_fwd_element_table", "radial_attn_bwd_element_table",
         "radial_attn_fwd_varlen_element_table", "radial_attn_bwd_varlen_element_table",
         "radial_error_string"])


def test_library_exports_every_declared_symbol():
    lib = radial.lib()
    for name in declared_symbols():
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", api.library_path()],
                         capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r"\bT (radial_\w+)", out))
    assert set(declared_symbols()) <= exported
    assert set(api._SIGNATURES) == set(declared_symbols())


def test_error_strings():
    lib = radial.lib()
    for code in (OK, INVALID, HEADDIM, CAPACITY, SHAPE, MISALIGNED, TOO_LARGE, HIP):
        s = lib.radial_error_string(code).decode()
        assert s and s != "unknown error code"
    assert lib.radial_error_string(12345).decode() == "unknown error code"


def dims(F, S, w0, block=128):
    nb, nnz = ctypes.c_int32(-9), ctypes.c_int64(-9)
    rc = radial.lib().radial_mask_dims(F, S, w0, block, ctypes.byref(nb), ctypes.byref(nnz))
    return rc, nb.value, nnz.value


def test_mask_dims_errors():
    assert dims(0, 10, 5)[0] == INVALID
    assert dims(4, 0, 5)[0] == INVALID
    assert dims(4, 10, 0)[0] == INVALID
    assert dims(4, 10, -3)[0] == INVALID
    assert dims(4, 10, 5, block=64)[0] == INVALID
    assert dims(1 << 16, 1 << 16, 5)[0] == TOO_LARGE
    assert radial.lib().radial_mask_dims(4, 10, 5, 128, None, None) == INVALID
    assert dims(4, 256, 256) == (OK, 8, 64)


def test_build_mask_errors():
    lib = radial.lib()
    rp = (ctypes.c_int32 * 9)()
    ci = (ctypes.c_int32 * 64)()
    assert lib.radial_build_mask(4, 256, 256, 128, None, ci, 64) == INVALID
    assert lib.radial_build_mask(4, 256, 256, 128, rp, None, 64) == INVALID
    assert lib.radial_build_mask(4, 256, 256, 128, rp, ci, -1) == INVALID
    assert lib.radial_build_mask(4, 256, 256, 128, rp, ci, 63) == CAPACITY
    assert lib.radial_build_mask(4, 256, 256, 100, rp, ci, 64) == INVALID
    assert lib.radial_build_mask(4, 256, 256, 128, rp, ci, 64) == OK
    assert list(rp) == list(range(0, 72, 8))
    with pytest.raises(radial.RadialError) as e:
        radial.build_mask(3, 100, 0)
    assert e.value.code == INVALID


def test_grid_mask_errors():
    lib = radial.lib()
    nb, nnz = ctypes.c_int32(-9), ctypes.c_int64(-9)
    args = (ctypes.byref(nb), ctypes.byref(nnz))
    assert lib.radial_mask_dims_grid(0, 30, 52, 81, 128, *args) == INVALID
    assert lib.radial_mask_dims_grid(4, 0, 52, 81, 128, *args) == INVALID
    assert lib.radial_mask_dims_grid(4, 30, -1, 81, 128, *args) == INVALID
    assert lib.radial_mask_dims_grid(4, 30, 52, 0, 128, *args) == INVALID
    assert lib.radial_mask_dims_grid(4, 30, 52, 81, 64, *args) == INVALID
    assert lib.radial_mask_dims_grid(1 << 10, 1 << 11, 1 << 11, 5, 128, *args) == TOO_LARGE
    assert lib.radial_mask_dims_grid(4, 30, 52, 81, 128, None, None) == INVALID
    assert lib.radial_mask_dims_grid(2, 16, 16, 31, 128, *args) == OK
    assert (nb.value, nnz.value) == (4, 16)  # W0 = 31 > 15 + 15: every block at any distance
    rp = (ctypes.c_int32 * 5)()
    ci = (ctypes.c_int32 * 16)()
    assert lib.radial_build_mask_grid(2, 16, 16, 31, 128, rp, ci, 15) == CAPACITY
    assert lib.radial_build_mask_grid(2, 16, 16, 31, 128, None, ci, 16) == INVALID
    assert lib.radial_build_mask_grid(2, 16, 16, 31, 128, rp, ci, 16) == OK
    assert list(rp) == [0, 4, 8, 12, 16]


def fwd(**kw):
    """Call radial_attn_fwd with valid-looking defaults, overridden by kw."""
    a = dict(q=0x10000, k=0x20000, v=0x30000, o=0x40000, lse=None, row_ptr=0x50000,
             col_idx=0x60000, nb=8, pairs=None, npairs=0, scale=0.125, elem_s=0, elem_w0=0,
             elem_gw=0, batch=1, heads=2,
             seqlen=1000, head_dim=128, stride_b=2 * 1000 * 128, stride_h=1000 * 128,
             stride_s=128, stream=None)
    a.update(kw)
    return radial.lib().radial_attn_fwd(
        a["q"], a["k"], a["v"], a["o"], a["lse"], a["row_ptr"], a["col_idx"], a["nb"],
        a["pairs"], a["npairs"], a["scale"], a["elem_s"], a["elem_w0"], a["elem_gw"],
        a["batch"], a["heads"], a["seqlen"],
        a["head_dim"], a["stride_b"], a["stride_h"], a["stride_s"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), INVALID), (dict(k=None), INVALID), (dict(v=None), INVALID),
    (dict(o=None), INVALID), (dict(row_ptr=None), INVALID), (dict(col_idx=None), INVALID),
    (dict(batch=0), INVALID), (dict(heads=-1), INVALID), (dict(seqlen=0), INVALID),
    (dict(nb=0), INVALID), (dict(scale=-0.5), INVALID), (dict(scale=float("nan")), INVALID),
    (dict(scale=float("inf")), INVALID), (dict(stride_s=64), INVALID),
    (dict(head_dim=96), HEADDIM), (dict(head_dim=256), HEADDIM),
    (dict(nb=9), SHAPE), (dict(nb=7), SHAPE),
    (dict(q=0x10008), MISALIGNED), (dict(o=0x40002), MISALIGNED),
    (dict(stride_s=132), MISALIGNED), (dict(stride_h=1000 * 128 + 4), MISALIGNED),
    (dict(batch=1 << 12, heads=1 << 12, seqlen=1 << 20, nb=1 << 13,
          stride_h=(1 << 20) * 128, stride_b=(1 << 32) * 128), TOO_LARGE),
    # The kernel's union list holds one 16-bit entry per key block: nb <= 16352.
    (dict(heads=1, seqlen=16353 * 128, nb=16353, stride_h=16353 * 128 * 128,
          stride_b=16353 * 128 * 128), TOO_LARGE),
    (dict(stride_s=(1 << 30) // 128 * 2), TOO_LARGE),  # a 128-row tile past 2^31 bytes
    # A pair table must hold between ceil(nb / 2) and nb pairs.
    (dict(pairs=0x70000, npairs=3), INVALID), (dict(pairs=0x70000, npairs=9), INVALID),
    (dict(pairs=0x70000, npairs=-1), INVALID),
    # Element masking needs a frame of one tile up to 2^22 tokens, W0 >= 1 and a grid
    # width of 0 or a divisor of the frame length.
    (dict(elem_s=100, elem_w0=50), INVALID), (dict(elem_s=-5, elem_w0=50), INVALID),
    (dict(elem_s=256, elem_w0=0), INVALID), (dict(elem_s=(1 << 22) + 1, elem_w0=5), INVALID),
    (dict(elem_s=1560, elem_w0=81, elem_gw=50), INVALID),
    (dict(elem_s=1560, elem_w0=81, elem_gw=-52), INVALID),
])
def test_attn_fwd_validation(kw, code):
    assert fwd(**kw) == code


def test_element_table_bytes():
    lib = radial.lib()
    out = ctypes.c_int64(-9)
    assert lib.radial_element_table_bytes(10, ctypes.byref(out)) == OK and out.value == 20480
    assert lib.radial_element_table_bytes(0, ctypes.byref(out)) == OK and out.value == 0
    assert lib.radial_element_table_bytes(-1, ctypes.byref(out)) == INVALID
    assert lib.radial_element_table_bytes(10, None) == INVALID
    assert lib.radial_element_table_bytes(1 << 31, ctypes.byref(out)) == TOO_LARGE


def build_table(**kw):
    """Call radial_build_element_table with valid-looking defaults, overridden by kw (every
    case below fails before the launch)."""
    a = dict(row_ptr=0x10000, col_idx=0x20000, nb=256, nnz=36720, elem_s=1560, elem_w0=1560,
             elem_gw=0, table=0x30000, table_bytes=36720 * 2048, stream=None)
    a.update(kw)
    return radial.lib().radial_build_element_table(
        a["row_ptr"], a["col_idx"], a["nb"], a["nnz"], a["elem_s"], a["elem_w0"], a["elem_gw"],
        a["table"], a["table_bytes"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(row_ptr=None), INVALID), (dict(col_idx=None), INVALID), (dict(table=None), INVALID),
    (dict(nb=0), INVALID), (dict(nnz=-1), INVALID),
    # The table holds element decisions: a frame length of 128 .. 2^22 tokens is needed.
    (dict(elem_s=0, elem_w0=0), INVALID), (dict(elem_s=100), INVALID),
    (dict(elem_w0=0), INVALID), (dict(elem_gw=7), INVALID), (dict(elem_gw=-52), INVALID),
    (dict(nb=16353), TOO_LARGE), (dict(nnz=1 << 31, table_bytes=1 << 50), TOO_LARGE),
    (dict(table_bytes=36720 * 2048 - 1), CAPACITY), (dict(table=0x30008), MISALIGNED),
])
def test_build_element_table_validation(kw, code):
    assert build_table(**kw) == code


def test_build_element_table_of_no_blocks_launches_nothing():
    assert build_table(nnz=0, table_bytes=0) == OK


def fwd_table(**kw):
    """Call radial_attn_fwd_element_table with valid-looking defaults, overridden by kw."""
    a = dict(q=0x10000, k=0x20000, v=0x30000, o=0x40000, lse=None, row_ptr=0x50000,
             col_idx=0x60000, nb=8, pairs=None, npairs=0, scale=0.125, table=0x70000,
             batch=1, heads=2, seqlen=1000, head_dim=128, stride_b=2 * 1000 * 128,
             stride_h=1000 * 128, stride_s=128, stream=None)
    a.update(kw)
    return radial.lib().radial_attn_fwd_element_table(
        a["q"], a["k"], a["v"], a["o"], a["lse"], a["row_ptr"], a["col_idx"], a["nb"],
        a["pairs"], a["npairs"], a["scale"], a["table"], a["batch"], a["heads"], a["seqlen"],
        a["head_dim"], a["stride_b"], a["stride_h"], a["stride_s"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(table=None), INVALID), (dict(table=0x70008), MISALIGNED),
    (dict(q=None), INVALID), (dict(row_ptr=None), INVALID), (dict(nb=9), SHAPE),
    (dict(head_dim=96), HEADDIM), (dict(scale=-1.0), INVALID), (dict(q=0x10008), MISALIGNED),
    (dict(pairs=0x80000, npairs=3), INVALID),
    (dict(heads=1, seqlen=16353 * 128, nb=16353, stride_h=16353 * 128 * 128,
          stride_b=16353 * 128 * 128), TOO_LARGE),
])
def test_attn_fwd_element_table_validation(kw, code):
    assert fwd_table(**kw) == code


def test_python_wrapper_checks_before_the_library():
    import torch
    q = torch.zeros(1, 1, 256, 64, dtype=torch.bfloat16)
    m = radial.dense_mask(256)
    with pytest.raises(ValueError):
        radial.attn_fwd(q, q, q, m)       # CPU tensors are refused
    with pytest.raises(TypeError):
        radial.attn_fwd(q.float(), q.float(), q.float(), m)
    with pytest.raises(ValueError):
        radial.attn_fwd(q, q[:, :, :128], q, m)


def bwd(**kw):
    """Call radial_attn_bwd with valid-looking defaults, overridden by kw."""
    a = dict(q=0x10000, k=0x20000, v=0x30000, o=0x40000, do=0x50000, lse=0x60000,
             dq=0x70000, dk=0x80000, dv=0x90000, delta=0xa0000, row_ptr=0xb0000,
             col_idx=0xc0000, col_ptr=0xd0000, row_idx=0xe0000, nb=8, scale=0.125,
             elem_s=0, elem_w0=0, elem_gw=0, batch=1, heads=2, seqlen=1000, head_dim=128,
             stride_b=2 * 1000 * 128, stride_h=1000 * 128, stride_s=128, stream=None)
    a.update(kw)
    return radial.lib().radial_attn_bwd(
        a["q"], a["k"], a["v"], a["o"], a["do"], a["lse"], a["dq"], a["dk"], a["dv"],
        a["delta"], a["row_ptr"], a["col_idx"], a["col_ptr"], a["row_idx"], a["nb"],
        a["scale"], a["elem_s"], a["elem_w0"], a["elem_gw"], a["batch"], a["heads"], a["seqlen"],
        a["head_dim"], a["stride_b"], a["stride_h"], a["stride_s"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    *[(dict(**{name: None}), INVALID) for name in (
        "q", "k", "v", "o", "do", "lse", "dq", "dk", "dv", "delta", "row_ptr", "col_idx",
        "col_ptr", "row_idx")],
    (dict(batch=0), INVALID), (dict(seqlen=0), INVALID), (dict(scale=-1.0), INVALID),
    (dict(elem_s=64, elem_w0=10), INVALID), (dict(elem_s=256, elem_w0=0), INVALID),
    (dict(elem_s=1560, elem_w0=81, elem_gw=7), INVALID), (dict(head_dim=96), HEADDIM), (dict(nb=9), SHAPE), (dict(stride_s=64), INVALID),
    (dict(dk=0x80008), MISALIGNED), (dict(lse=0x60002), MISALIGNED),
    (dict(delta=0xa0001), MISALIGNED), (dict(stride_s=132), MISALIGNED),
    (dict(batch=1 << 12, heads=1 << 12, seqlen=1 << 20, nb=1 << 13,
          stride_h=(1 << 20) * 128, stride_b=(1 << 32) * 128), TOO_LARGE),
])
def test_attn_bwd_validation(kw, code):
    assert bwd(**kw) == code


def bwd_table(**kw):
    """Call radial_attn_bwd_element_table with valid-looking defaults, overridden by kw."""
    a = dict(q=0x10000, k=0x20000, v=0x30000, o=0x40000, do=0x50000, lse=0x60000,
             dq=0x70000, dk=0x80000, dv=0x90000, delta=0xa0000, row_ptr=0xb0000,
             col_idx=0xc0000, col_ptr=0xd0000, row_idx=0xe0000, nb=8, scale=0.125,
             table=0xf0000, batch=1, heads=2, seqlen=1000, head_dim=128,
             stride_b=2 * 1000 * 128, stride_h=1000 * 128, stride_s=128, stream=None)
    a.update(kw)
    return radial.lib().radial_attn_bwd_element_table(
        a["q"], a["k"], a["v"], a["o"], a["do"], a["lse"], a["dq"], a["dk"], a["dv"],
        a["delta"], a["row_ptr"], a["col_idx"], a["col_ptr"], a["row_idx"], a["nb"],
        a["scale"], a["table"], a["batch"], a["heads"], a["seqlen"], a["head_dim"],
        a["stride_b"], a["stride_h"], a["stride_s"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(table=None), INVALID), (dict(table=0xf0008), MISALIGNED),
    (dict(dq=None), INVALID), (dict(col_ptr=None), INVALID), (dict(nb=9), SHAPE),
    (dict(head_dim=96), HEADDIM), (dict(scale=float("nan")), INVALID),
    (dict(delta=0xa0001), MISALIGNED),
])
def test_attn_bwd_element_table_validation(kw, code):
    assert bwd_table(**kw) == code


def test_transpose_mask_errors_and_a_small_case():
    import ctypes
    lib = radial.lib()
    rp = (ctypes.c_int32 * 4)(0, 2, 3, 5)
    ci = (ctypes.c_int32 * 5)(0, 2, 1, 0, 7)  # 7 is outside [0, 3): dropped
    cp = (ctypes.c_int32 * 4)()
    ri = (ctypes.c_int32 * 5)()
    assert lib.radial_transpose_mask(3, rp, ci, cp, ri) == OK
    assert list(cp) == [0, 2, 3, 4] and list(ri)[:4] == [0, 2, 1, 0]
    assert lib.radial_transpose_mask(0, rp, ci, cp, ri) == INVALID
    assert lib.radial_transpose_mask(3, None, ci, cp, ri) == INVALID
    assert lib.radial_transpose_mask(3, rp, None, cp, ri) == INVALID
    assert lib.radial_transpose_mask(3, rp, ci, None, ri) == INVALID
    assert lib.radial_transpose_mask(3, rp, ci, cp, None) == INVALID
    bad = (ctypes.c_int32 * 4)(0, 3, 2, 5)
    assert lib.radial_transpose_mask(3, bad, ci, cp, ri) == INVALID


def test_transpose_mask_matches_oracle():
    import numpy as np
    from oracle import radial_oracle as ro
    rng = np.random.default_rng(7)
    m = rng.random((37, 37)) < 0.25
    rp, ci = ro.csr(m)
    mask = radial.Mask(torch_int(rp), torch_int(ci), 1, 37 * 128, 1).transposed()
    cp, ri = ro.transpose_csr(rp, ci, 37)
    assert mask.col_ptr.tolist() == cp.tolist() and mask.row_idx.tolist() == ri.tolist()


def torch_int(x):
    import torch
    return torch.from_numpy(x.astype("int32"))


def varlen(**kw):
    """Call radial_attn_fwd_varlen with valid-looking defaults, overridden by kw."""
    import ctypes
    a = dict(q=0x10000, k=0x20000, v=0x30000, o=0x40000, lse=None, seq=[1000, 300], batch=2,
             row_ptr=0x50000, col_idx=0x60000, pairs=None, npairs=None, scale=0.125,
             elem_s=0, elem_w0=0, elem_gw=0, heads=2, head_dim=128, stride_h=128, stride_s=256,
             stream=None)
    a.update(kw)
    seq = None if a["seq"] is None else (ctypes.c_int32 * len(a["seq"]))(*a["seq"])
    npr = None if a["npairs"] is None else (ctypes.c_int32 * len(a["npairs"]))(*a["npairs"])
    return radial.lib().radial_attn_fwd_varlen(
        a["q"], a["k"], a["v"], a["o"], a["lse"], seq, a["batch"], a["row_ptr"], a["col_idx"],
        a["pairs"], npr, a["scale"], a["elem_s"], a["elem_w0"], a["elem_gw"], a["heads"],
        a["head_dim"],
        a["stride_h"], a["stride_s"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), INVALID), (dict(row_ptr=None), INVALID), (dict(seq=None), INVALID),
    (dict(batch=0), INVALID), (dict(seq=[1000, 0]), INVALID), (dict(heads=0), INVALID),
    (dict(pairs=0x70000), INVALID),                              # pairs without counts
    (dict(pairs=0x70000, npairs=[9, 2]), INVALID),               # 9 pairs for 8 blocks
    (dict(pairs=0x70000, npairs=[3, 2]), INVALID),               # 3 < ceil(8 / 2)
    (dict(stride_s=64), INVALID), (dict(scale=float("nan")), INVALID),
    (dict(elem_s=64, elem_w0=5), INVALID), (dict(elem_s=300, elem_w0=5, elem_gw=7), INVALID),
    (dict(head_dim=80), HEADDIM),
    (dict(v=0x30004), MISALIGNED), (dict(stride_h=132), MISALIGNED),
    (dict(seq=[100] * 65, batch=65), TOO_LARGE),
    (dict(seq=[16353 * 128], batch=1), TOO_LARGE),
])
def test_attn_fwd_varlen_validation(kw, code):
    # Every case here fails a host check: none may reach a launch (the pointers are fake).
    assert varlen(**kw) == code


def rule(**kw):
    """Call radial_attn_fwd_rule with valid-looking defaults, overridden by kw."""
    a = dict(q=0x10000, k=0x20000, v=0x30000, o=0x40000, lse=None, frames=4, s=250, gw=0,
             w0=100, element=0, pairs=None, npairs=0, scale=0.125, batch=1, heads=2,
             head_dim=128, stride_b=2 * 1000 * 128, stride_h=1000 * 128, stride_s=128,
             stream=None)
    a.update(kw)
    return radial.lib().radial_attn_fwd_rule(
        a["q"], a["k"], a["v"], a["o"], a["lse"], a["frames"], a["s"], a["gw"], a["w0"],
        a["element"], a["pairs"], a["npairs"], a["scale"], a["batch"], a["heads"],
        a["head_dim"], a["stride_b"], a["stride_h"], a["stride_s"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), INVALID), (dict(o=None), INVALID), (dict(frames=0), INVALID),
    (dict(s=0), INVALID), (dict(w0=0), INVALID), (dict(gw=-1), INVALID),
    (dict(gw=7), INVALID),                                   # 7 does not divide 250
    (dict(batch=0), INVALID), (dict(heads=0), INVALID), (dict(scale=-1.0), INVALID),
    (dict(stride_s=64), INVALID), (dict(head_dim=96), HEADDIM),
    (dict(q=0x10008), MISALIGNED), (dict(stride_h=1000 * 128 + 4), MISALIGNED),
    (dict(element=1, s=100, frames=10), INVALID),            # element: frame below 128
    (dict(pairs=0x70000, npairs=3), INVALID), (dict(pairs=0x70000, npairs=9), INVALID),
    (dict(frames=16353, s=128), TOO_LARGE),                  # past 16352 blocks
    (dict(frames=300000, s=1), TOO_LARGE),                   # 2 x 300000 marking steps a row
    (dict(frames=100, s=2000, gw=2), TOO_LARGE),             # 2 x 100 x 1000 steps a row
    (dict(frames=1 << 16, s=1 << 16), TOO_LARGE),
])
def test_attn_fwd_rule_validation(kw, code):
    assert rule(**kw) == code


def bwd_varlen(**kw):
    """Call radial_attn_bwd_varlen with valid-looking defaults, overridden by kw."""
    import ctypes
    a = dict(q=0x10000, k=0x20000, v=0x30000, o=0x40000, do=0x50000, lse=0x60000,
             dq=0x70000, dk=0x80000, dv=0x90000, delta=0xa0000, seq=[1000, 300], batch=2,
             row_ptr=0xb0000, col_idx=0xc0000, col_ptr=0xd0000, row_idx=0xe0000,
             scale=0.125, elem_s=0, elem_w0=0, elem_gw=0, heads=2, head_dim=128,
             stride_h=128, stride_s=256, stream=None)
    a.update(kw)
    seq = None if a["seq"] is None else (ctypes.c_int32 * len(a["seq"]))(*a["seq"])
    return radial.lib().radial_attn_bwd_varlen(
        a["q"], a["k"], a["v"], a["o"], a["do"], a["lse"], a["dq"], a["dk"], a["dv"],
        a["delta"], seq, a["batch"], a["row_ptr"], a["col_idx"], a["col_ptr"], a["row_idx"],
        a["scale"], a["elem_s"], a["elem_w0"], a["elem_gw"], a["heads"], a["head_dim"],
        a["stride_h"], a["stride_s"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    *[(dict(**{name: None}), INVALID) for name in (
        "q", "k", "v", "o", "do", "lse", "dq", "dk", "dv", "delta", "seq", "row_ptr",
        "col_idx", "col_ptr", "row_idx")],
    (dict(batch=0), INVALID), (dict(seq=[1000, 0]), INVALID), (dict(heads=0), INVALID),
    (dict(scale=float("nan")), INVALID), (dict(stride_s=64), INVALID),
    (dict(elem_s=64, elem_w0=5), INVALID), (dict(elem_s=300, elem_w0=5, elem_gw=7), INVALID),
    (dict(head_dim=80), HEADDIM), (dict(dk=0x80004), MISALIGNED),
    (dict(delta=0xa0002), MISALIGNED), (dict(stride_h=132), MISALIGNED),
    (dict(seq=[100] * 65, batch=65), TOO_LARGE),
])
def test_attn_bwd_varlen_validation(kw, code):
    # Every case here fails a host check: none may reach a launch (the pointers are fake).
    assert bwd_varlen(**kw) == code


def varlen_rule(**kw):
    """Call radial_attn_fwd_varlen_rule with valid-looking defaults, overridden by kw."""
    import ctypes
    a = dict(q=0x10000, k=0x20000, v=0x30000, o=0x40000, lse=None, frames=[4, 2], batch=2,
             s=250, gw=0, w0=100, element=0, pairs=None, npairs=None, scale=0.125, heads=2,
             head_dim=128, stride_h=128, stride_s=256, stream=None)
    a.update(kw)
    fr = None if a["frames"] is None else (ctypes.c_int32 * len(a["frames"]))(*a["frames"])
    npr = None if a["npairs"] is None else (ctypes.c_int32 * len(a["npairs"]))(*a["npairs"])
    return radial.lib().radial_attn_fwd_varlen_rule(
        a["q"], a["k"], a["v"], a["o"], a["lse"], fr, a["batch"], a["s"], a["gw"], a["w0"],
        a["element"], a["pairs"], npr, a["scale"], a["heads"], a["head_dim"], a["stride_h"],
        a["stride_s"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), INVALID), (dict(frames=None), INVALID), (dict(batch=0), INVALID),
    (dict(frames=[4, 0]), INVALID), (dict(s=0), INVALID), (dict(w0=0), INVALID),
    (dict(gw=7), INVALID), (dict(gw=-1), INVALID), (dict(heads=0), INVALID),
    (dict(element=1, s=100), INVALID), (dict(pairs=0x70000), INVALID),
    (dict(pairs=0x70000, npairs=[9, 2]), INVALID), (dict(head_dim=80), HEADDIM),
    (dict(stride_h=132), MISALIGNED), (dict(frames=[1] * 65, batch=65), TOO_LARGE),
    (dict(frames=[16353, 1], s=128), TOO_LARGE), (dict(frames=[300000, 1], s=1), TOO_LARGE),
])
def test_attn_fwd_varlen_rule_validation(kw, code):
    # Every case here fails a host check: none may reach a launch (the pointers are fake).
    assert varlen_rule(**kw) == code


def varlen_tables(**kw):
    """Call the two varlen element-table entry points with valid-looking defaults."""
    import ctypes
    a = dict(q=0x10000, k=0x20000, v=0x30000, o=0x40000, lse=0x60000, do=0x50000,
             dq=0x70000, dk=0x80000, dv=0x90000, delta=0xa0000, seq=[1000, 300], batch=2,
             row_ptr=0xb0000, col_idx=0xc0000, col_ptr=0xd0000, row_idx=0xe0000, pairs=None,
             npairs=None, scale=0.125, table=0xf0000, heads=2, head_dim=128, stride_h=128,
             stride_s=256, stream=None)
    a.update(kw)
    seq = None if a["seq"] is None else (ctypes.c_int32 * len(a["seq"]))(*a["seq"])
    lib = radial.lib()
    f = lib.radial_attn_fwd_varlen_element_table(
        a["q"], a["k"], a["v"], a["o"], a["lse"], seq, a["batch"], a["row_ptr"], a["col_idx"],
        a["pairs"], a["npairs"], a["scale"], a["table"], a["heads"], a["head_dim"],
        a["stride_h"], a["stride_s"], a["stream"])
    b = lib.radial_attn_bwd_varlen_element_table(
        a["q"], a["k"], a["v"], a["o"], a["do"], a["lse"], a["dq"], a["dk"], a["dv"],
        a["delta"], seq, a["batch"], a["row_ptr"], a["col_idx"], a["col_ptr"], a["row_idx"],
        a["scale"], a["table"], a["heads"], a["head_dim"], a["stride_h"], a["stride_s"],
        a["stream"])
    return f, b


@pytest.mark.parametrize("kw,code", [
    (dict(table=None), INVALID), (dict(table=0xf0004), MISALIGNED), (dict(q=None), INVALID),
    (dict(seq=None), INVALID), (dict(batch=0), INVALID), (dict(head_dim=80), HEADDIM),
    (dict(scale=-2.0), INVALID), (dict(stride_h=132), MISALIGNED),
    (dict(seq=[100] * 65, batch=65), TOO_LARGE),
])
def test_varlen_element_table_validation(kw, code):
    assert varlen_tables(**kw) == (code, code)
