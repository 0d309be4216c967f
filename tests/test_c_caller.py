"""The boundary from plain C: tests/c_caller/caller.c includes include/radial_attn.h,
compiles as pedantic C99, links against libradial.so and calls host entry points (no
GPU needed). The mask sizes it prints are the survey's Wan figures (nb = 256, 36,720
active blocks) and the library's own."""
import os
import subprocess

import block_sparse_attention_radial_amd as radial
from block_sparse_attention_radial_amd import api

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_c99_caller(tmp_path):
    lib = api.library_path()
    radial.lib()  # built
    exe = str(tmp_path / "caller")
    cmd = ["gcc", "-std=c99", "-Wall", "-Wextra", "-pedantic", "-Werror",
           f"-I{os.path.join(ROOT, 'include')}", os.path.join(ROOT, "tests", "c_caller", "caller.c"),
           lib, f"-Wl,-rpath,{os.path.dirname(lib)}", "-o", exe]
    res = subprocess.run(cmd, capture_output=True, text=True, timeout=120)
    assert res.returncode == 0, res.stderr
    run = subprocess.run([exe], capture_output=True, text=True, timeout=60,
                         env=dict(os.environ, HIP_VISIBLE_DEVICES=""))
    assert run.returncode == 0, run.stderr
    m = radial.build_mask(21, 1560, 1560, pairs=False)
    last = int(m.row_ptr[-1] - m.row_ptr[-2])
    assert run.stdout.strip() == (
        f"nb=256 nnz=36720 last_row={last} table_bytes={36720 * 2048} "
        f"err={radial.error_string(-4)}")
