"""bench.py's command-line contract that needs no GPU: it measures one GPU
only, so a multi-GPU request exits non-zero with a message saying so, before
touching a device; and the roofline byte counts it reports follow the
algorithmic definitions."""

import os
import subprocess
import sys

from conftest import ROOT


def run_bench(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, cwd=ROOT, timeout=120)


def test_more_than_one_gpu_is_refused():
    r = run_bench("--gpus", "2", "--no-cpu")
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_world_size_above_one_is_refused():
    env = dict(os.environ, WORLD_SIZE="4")
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--no-cpu"],
                       capture_output=True, text=True, cwd=ROOT, timeout=120, env=env)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_gemm_bytes_match_the_layout():
    """Codes + headers + X + Y of one 70B-class up-projection call."""
    from bit_weight_only_wq_amd import roofline as rl
    N, K, G = 28672, 8192, 128
    for B in (1, 16, 64):
        expect = N * K // 2 + 4 * N * (K // G) + 2 * B * K + 2 * B * N
        assert rl.gemm_bytes(B, N, K, G, 4) == expect
