"""Build libradial.so in-tree with hipcc for gfx950.

    python -m block_sparse_attention_radial_amd.build

The library lands in block_sparse_attention_radial_amd/lib/libradial.so. It holds the
host mask builder and the gfx950 kernels behind the C ABI of include/radial_attn.h.
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB_DIR = os.path.join(PKG, "lib")
LIB_PATH = os.path.join(LIB_DIR, "libradial.so")
SOURCES = ["radial_mask.cpp", "radial_pairs.cpp", "radial_attn_fwd.hip", "radial_attn_bwd.hip"]
ARCH = "gfx950"


def hipcc_path() -> str:
    return os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def compile_flags() -> list[str]:
    return [
        f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
        f"-I{os.path.join(ROOT, 'include')}",
        # Packed fp32 VALU forms stay off; ordinary fp32 code is emitted instead.
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    ]


def build(verbose: bool = False) -> str:
    """Compile every source into libradial.so (always recompiles). Returns its path."""
    os.makedirs(LIB_DIR, exist_ok=True)
    tmp = LIB_PATH + f".tmp{os.getpid()}"
    cmd = [hipcc_path(), *compile_flags(), *(os.path.join(CSRC, s) for s in SOURCES), "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the gfx950-only feature above and says so; that
    # line is noise, anything else is shown.
    noise = "is not a recognized feature for this target"
    msgs = [ln for ln in (res.stdout + res.stderr).splitlines() if noise not in ln]
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if msgs and verbose:
        print("\n".join(msgs), flush=True)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
