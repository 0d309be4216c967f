"""Write tests/golden/masks.json: block-mask summaries computed by the CPU oracle alone.

Run from the repository root:  python tests/golden/make_golden.py
Each case stores the CSR size, the per-row extremes and a SHA-256 of the int32
little-endian row_ptr followed by col_idx. Nothing here comes from the HIP path.
"""
import hashlib
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)
from oracle import radial_oracle as ro  # noqa: E402

CASES = [
    # name, frames, tokens_per_frame, w0, grid width (None: the 1-D distance)
    ("tiny", 4, 256, 256, None),
    ("small", 8, 1024, 512, None),
    ("wan2.1-14b-shaped", 21, 1560, 1560, None),
    ("hunyuanvideo-shaped", 33, 3600, 3600, None),
    ("4x-long-wan-shaped", 84, 1560, 1560, None),
    ("ragged-sparse", 6, 1000, 100, None),
    ("ragged-half", 8, 1000, 334, None),
    ("short-frames", 12, 100, 37, None),
    # the 2-D grid distance: Wan's 30 x 52 and HunyuanVideo's 45 x 80 token grids
    ("wan2.1-14b-shaped-grid", 21, 1560, 81, 52),
    ("hunyuanvideo-shaped-grid", 33, 3600, 124, 80),
    ("grid-rows-of-8", 9, 200, 7, 8),
]


def main():
    out = []
    for name, F, S, w0, gw in CASES:
        counts = ro.block_counts(F, S, w0, grid_w=gw)
        row_ptr, col_idx = ro.csr(counts > 0)
        h = hashlib.sha256()
        h.update(row_ptr.astype("<i4").tobytes())
        h.update(col_idx.astype("<i4").tobytes())
        per_row = np.diff(row_ptr)
        extra = {} if gw is None else {"grid_w": gw}
        out.append(dict(name=name, frames=F, tokens_per_frame=S, w0=w0, **extra, n=F * S,
                        nb=len(row_ptr) - 1, nnz=int(row_ptr[-1]),
                        row_nnz_min=int(per_row.min()), row_nnz_max=int(per_row.max()),
                        allowed_elements=int(counts.sum()), sha256=h.hexdigest()))
        print(out[-1], flush=True)
    with open(os.path.join(os.path.dirname(os.path.abspath(__file__)), "masks.json"), "w") as f:
        json.dump({"generator": "tests/golden/make_golden.py (CPU oracle only)",
                   "cases": out}, f, indent=1)
        f.write("\n")


if __name__ == "__main__":
    main()
