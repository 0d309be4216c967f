"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer (no GPU).

tests/sanitize/host_sweep.cpp drives every C entry point through its host paths: the
mask builders on a seeded sweep of 1-D and grid shapes (exact-size heap buffers, and a
col_idx one entry short for the capacity error), the pair table, the transpose, and the
argument checks of every attention and element-table entry point, which return before
any HIP call (a
call that passes them fails at its first HIP call here, with RADIAL_ERR_HIP). The
library sources are compiled with the sanitizers on the host side only; the device code
is built as usual and never runs.
"""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "block_sparse_attention_radial_amd", "csrc")
SOURCES = [os.path.join(CSRC, f) for f in
           ("radial_mask.cpp", "radial_pairs.cpp", "radial_attn_fwd.hip", "radial_attn_bwd.hip")]
DRIVER = os.path.join(ROOT, "tests", "sanitize", "host_sweep.cpp")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


@pytest.fixture(scope="module")
def sweep_binary(tmp_path_factory):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc is not installed")
    out = str(tmp_path_factory.mktemp("sanitize") / "host_sweep")
    cmd = [HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17",
           "-fno-omit-frame-pointer",
           "-Xarch_host", "-fsanitize=address",
           "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           f"-I{os.path.join(ROOT, 'include')}", *SOURCES, DRIVER, "-o", out]
    res = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert res.returncode == 0, res.stderr[-4000:]
    return out


def test_host_code_is_clean_under_asan_and_ubsan(sweep_binary):
    env = dict(os.environ,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:exitcode=23",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1",
               HIP_VISIBLE_DEVICES="")
    res = subprocess.run([sweep_binary], capture_output=True, text=True, timeout=600, env=env)
    report = res.stdout[-4000:] + res.stderr[-4000:]
    assert res.returncode == 0, report
    assert "AddressSanitizer" not in res.stderr and "runtime error" not in res.stderr, report
    assert res.stdout.strip().startswith("OK "), report
