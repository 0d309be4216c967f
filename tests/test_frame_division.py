"""The frame split the kernel's element masking uses, checked exhaustively on the CPU.

For a token index a < 2^21 (the kernel's sequence limit is 16352 blocks of 128) and a
frame length S >= 128, the kernel forms q = trunc(float32(a) * r) with r an approximate
float32 reciprocal of S (v_rcp_f32, within a few ulp), then corrects q by one in either
direction from the remainder. This test emulates those float32 steps with numpy and
checks (q, a - qS) against integer division, for every a < 2^21, for reciprocals up to
+-2 ulp off, and for frame lengths from 128 up to 2^21. The grid distance splits an
in-frame index (also below 2^21) by the grid width the same way, so widths from 1 up
are checked too.
"""
import numpy as np
import pytest

A = np.arange(0, 1 << 21, dtype=np.int64)
A32 = A.astype(np.float32)

FRAMES = [128, 129, 130, 255, 256, 300, 1000, 1024, 1560, 3600, 4095, 65535, 1 << 20,
          (1 << 21) - 1]


GRID_WIDTHS = [1, 2, 3, 5, 7, 8, 13, 31, 52, 80, 97, 127]


@pytest.mark.parametrize("S", FRAMES + GRID_WIDTHS +
                         np.random.default_rng(0).integers(128, 1 << 21, 12).tolist())
def test_float_quotient_with_one_correction_is_exact(S):
    base = np.float32(1.0) / np.float32(S)
    for ulp in range(-2, 3):
        r = base
        for _ in range(abs(ulp)):
            r = np.nextafter(r, np.float32(np.inf if ulp > 0 else 0.0), dtype=np.float32)
        q = (A32 * r).astype(np.float32).astype(np.int64)  # truncation; a >= 0
        rem = A - q * S
        up = rem >= S
        q[up] += 1
        rem[up] -= S
        down = rem < 0
        q[down] -= 1
        rem[down] += S
        assert np.array_equal(q, A // S) and np.array_equal(rem, A % S), (S, ulp)
