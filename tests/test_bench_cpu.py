"""Host-side checks of bench.py's contract that need no GPU."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300)
    assert r.returncode != 0
    assert "one MI355X" in (r.stdout + r.stderr)


def test_algorithmic_counts():
    # the per-launch work the roofline divides by: 2 HI dI flop per visible (query, entry) pair,
    # and the decode scoring's key, query, weight and score bytes
    sys.path.insert(0, ROOT)
    import bench
    from compressed_sparse_kv_02_amd import layer as LY
    L = LY.chunked_prefill_512k()[0]
    pairs = sum(min(L.N, (L.pos0 + j + 1) // L.m) for j in range(L.T)) * L.batch
    assert bench.indexer_flops(L) == 2 * L.HI * L.dI * pairs
