"""The measurement harness on the host: its one-GPU refusal, the algorithmic
bytes it divides by, and the tie between counter summaries and kernel sources."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120, cwd=ROOT)
    assert r.returncode != 0
    assert "one GPU" in r.stdout + r.stderr


def test_algorithmic_bytes_of_the_main_workload():
    """36 x 16 x 8 segments of 32768 bf16 keys at head_dim 128, B = 2048: every
    key's K row read once, the kept K and V rows read and written, the kept
    positions read and written."""
    n_seg, N, B, d, es = 36 * 16 * 8, 32768, 2048, 128, 2
    score, gather = bench.algorithmic_bytes(n_seg * N, n_seg, n_seg * B, d, es)
    assert score == n_seg * N * d * es == 38654705664
    assert gather == n_seg * B * (4 * d * es + 8) == 9739173888
    assert score + gather == 48393879552


def test_counter_summaries_follow_their_sources():
    """A summary counts only for the sources it was taken on: the hash covers
    the kernel's own file and the shared ones, and changes with any of them."""
    for k in bench.KERNEL_SOURCE:
        h = bench.kernel_source_sha(k)
        assert len(h) == 16 and h == bench.kernel_source_sha(k)
    assert bench.kernel_source_sha("score") != bench.kernel_source_sha("select_gather")
    assert bench.read_traffic("score", "no_such_workload") is None
