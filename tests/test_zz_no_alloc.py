"""radial_attn_bwd_noalloc against radial_attn_bwd, through the C ABI (GPU).

The allocation-free entry point keeps the backward's workspace (D_i and the base-2 lse)
in the library's static device memory instead of a caller buffer. Its gradients must equal those of
radial_attn_bwd (the same kernels) bit for bit: on two calls in a row, the second with a
smaller input, so that the second call runs on the workspace the first one left behind.
A shape past the workspace is refused.
"""
import ctypes

import pytest
import torch

import block_sparse_attention_radial_amd as radial
from block_sparse_attention_radial_amd.inputs import Workload, draw_qkv

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    radial.lib()


def case(wl, seed, element=False):
    q, k, v = (x.cuda() for x in draw_qkv(wl, seed=seed))
    g = torch.Generator(device="cuda").manual_seed(seed + 1)
    do = torch.randn(q.shape, generator=g, device="cuda").to(torch.bfloat16)
    mask = radial.build_mask(wl.frames, wl.tokens_per_frame, wl.w0).transposed().to("cuda")
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device="cuda")
    o = radial.attn_fwd(q, k, v, mask, lse=lse, element=element)
    return q, k, v, o, do, lse, mask


def test_noalloc_equals_attn_bwd_on_two_calls():
    big = Workload("big", 2, 3, 128, 6, 1560, 1560, 1.0)
    small = Workload("small", 1, 2, 64, 5, 1000, 300, 1.0)
    for wl, element in ((big, False), (small, True)):
        q, k, v, o, do, lse, mask = case(wl, seed=wl.n, element=element)
        ref = radial.attn_bwd(q, k, v, o, do, lse, mask, element=element)
        out = tuple(torch.full_like(q, float("nan")) for _ in range(3))
        got = radial.attn_bwd_noalloc(q, k, v, o, do, lse, mask, element=element, out=out)
        torch.cuda.synchronize()
        for a, b in zip(got, ref):
            assert torch.equal(a, b), wl.name


def test_noalloc_refuses_a_shape_past_the_workspace():
    lib = radial.lib()
    fake = ctypes.c_void_p(256)  # never dereferenced: the size check comes first
    rc = lib.radial_attn_bwd_noalloc(*([fake] * 13), 2048, 0.1, 0, 0, 0, 1, 33, 2**18, 128,
                                     0, 0, 128, None)
    assert rc == -6  # RADIAL_ERR_TOO_LARGE: 33 * 2^18 rows > 2^23
