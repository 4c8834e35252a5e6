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


def _bench_module():
    sys.path.insert(0, ROOT)
    import bench
    return bench


def test_committed_counter_and_traffic_summaries_match_the_sources():
    """The profiles the bench line reads (per-launch HBM traffic, matrix-core
    busy share per batch size) were taken on the kernel sources as they are:
    their recorded source hashes match, so the bench reports them instead of
    null."""
    bench = _bench_module()
    w = "mlp70b_up_k8192_n28672_g128"
    for B in (1, 16, 64):
        assert bench.read_traffic(f"wq_gemm_b{B}_{w}") is not None, B
    busy = bench.read_mfma_counters(w)
    assert sorted(busy) == [1, 2, 4, 8, 16, 32, 64]
    assert busy[1] == 0.0 and all(0.0 < busy[B] < 1.0 for B in (2, 4, 8, 16, 32, 64))


def test_counter_summary_with_other_sources_is_ignored(tmp_path):
    """A counter summary whose source hash does not match is not used."""
    bench = _bench_module()
    text = open(os.path.join(ROOT, "profiles", "mfma_counters_wq_gemm_mlp70b_up_k8192_n28672_g128.txt")).read()
    lines = [("sources_sha256: " + "0" * 64) if l.startswith("sources_sha256:") else l for l in text.splitlines()]
    p = tmp_path / "mfma_counters.txt"
    p.write_text("\n".join(lines))
    assert bench.read_mfma_counters("x", path=str(p)) == {}
    p.write_text(text)
    assert bench.read_mfma_counters("x", path=str(p))[64] > 0.0
