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


def test_decode_step_and_attention_counts():
    sys.path.insert(0, ROOT)
    import bench
    from compressed_sparse_kv_02_amd import layer as LY
    csa, hca = LY.decode_1m()
    # indexer keys 8 x 262144 x 128 x 2 B dominate; HCA entries 8 x 8192 x 1 KiB; selected rows
    # 8 x 1024 x 1 KiB; about 617 MB in all
    sb = bench.decode_step_bytes([csa, hca])
    assert 8 * 262144 * 256 + 8 * 8192 * 1024 + 8 * 1024 * 1024 < sb < 0.62e9
    assert bench.decode_score_bytes(csa) == 8 * (262144 * 256 + 64 * 256 + 64 * 4)
    # a 3-token toy: pairs = selected-or-visible entries + window rows per query
    L = LY.LayerCall("hca", 1, 3, 8, 2, d=64, H=2, m=4, w=2)
    # t = 8, 9, 10: V = 2, 2, 2 (N = 2); window min(2, t + 1) = 2 each
    assert bench.attn_pairs(L) == 3 * (2 + 2) and bench.attn_flops(L) == 4 * 2 * 64 * 12
    Lc = LY.LayerCall("csa", 1, 3, 8, 2, d=64, H=2, m=4, w=2, k=1)
    assert bench.attn_pairs(Lc) == 3 * (1 + 2)
