"""bench.py's command-line contract, checked without a GPU.

More than one GPU is refused with a message (the benchmark measures one GPU); a run on a
host without a GPU exits with an error instead of printing a result line; the traffic
record is keyed to the kernel sources.
"""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BENCH = os.path.join(ROOT, "bench.py")


def run(*args, env=None):
    return subprocess.run([sys.executable, BENCH, *args], capture_output=True, text=True,
                          timeout=300, env=env, cwd=ROOT)


def test_more_than_one_gpu_is_refused():
    r = run("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


def test_world_size_above_one_is_refused():
    r = run(env=dict(os.environ, WORLD_SIZE="4"))
    assert r.returncode == 2 and r.stdout.strip() == ""


def test_no_gpu_means_no_result_line():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    r = run("--steps", "1", "--warmup", "0")
    assert r.returncode != 0
    assert r.stdout.strip() == ""


def test_help_lists_every_leg():
    r = run("--help")
    assert r.returncode == 0
    for flag in ("--element", "--backward", "--rule", "--varlen", "--workload"):
        assert flag in r.stdout


def test_traffic_record_follows_the_kernel_sources():
    sys.path.insert(0, ROOT)
    import bench
    digest = bench.kernel_digest()
    assert len(digest) == 64
    for name in ("wan2.1-14b-shaped", "4x-long-wan-shaped"):
        path = os.path.join(ROOT, "profiles", f"traffic_{name}.json")
        with open(path) as f:
            rec = json.load(f)
        got = bench.traffic_bytes(name)
        if rec["kernel_sha256"] == digest:
            assert got == rec["bytes_per_launch"] and got > 0
        else:  # counters taken on other sources are not reported
            assert got is None
    assert bench.traffic_bytes("no-such-workload") is None
