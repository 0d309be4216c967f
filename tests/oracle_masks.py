"""The oracle's own block masks, for the oracle side of the GPU parity tests.

The oracle walks the CSR that it builds from the rule itself (block_mask, then csr),
never the library's: the two builders are compared bit for bit in test_mask_builder.py,
and the parity tests then stay independent of that comparison. Cached, because several
tests reuse one shape.
"""
import functools

from oracle import radial_oracle as ro


@functools.lru_cache(maxsize=64)
def oracle_csr(frames: int, tokens_per_frame: int, w0: int, grid_w=None):
    """(row_ptr, col_idx) of the radial block mask, as built by the oracle."""
    rp, ci = ro.csr(ro.block_mask(frames, tokens_per_frame, w0, grid_w=grid_w))
    rp.flags.writeable = False
    ci.flags.writeable = False
    return rp, ci
