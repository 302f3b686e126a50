"""bench.py's command line without a GPU: more than one GPU is refused with a
message (one GPU is measured; sharding is design only), and the rocprofv3
summaries under profiles/ parse back into the figures the bench reports."""

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    env = dict(os.environ, WORLD_SIZE="4")
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")], capture_output=True, text=True, cwd=ROOT,
                       env=env)
    assert r.returncode == 2 and "one GPU" in r.stderr


def test_traffic_summary_matches_sources():
    """The counter summary of the headline kernel belongs to the current
    kernel sources (same hash), and its bytes are at least the algorithmic
    minimum of the launch (Q, K, V read once, O and LSE written once)."""
    sys.path.insert(0, ROOT)
    import bench
    t = bench.traffic_for_kernel()
    assert t is not None, "profiles/ counters were taken for other kernel sources"
    B, H, N, d = 4, 16, 4096, 128
    minimum = 4 * B * H * N * d * 2 + 4 * B * H * N
    assert minimum <= t <= 1.05 * minimum
