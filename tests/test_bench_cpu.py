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


def test_kernel_table_from_a_trace(tmp_path):
    # one line per library kernel and launch grid, torch's own kernels left out, times in us
    p = tmp_path / "run_kernel_trace.csv"
    rows = [("void cskv::attn_mfma<512, 4, 1, -1, 1>(cskv::AttnArgs)", 256, 144, 1, 1000, 25000),
            ("void cskv::attn_mfma<512, 4, 1, -1, 1>(cskv::AttnArgs)", 256, 144, 1, 30000, 53000),
            ("void cskv::attn_merge<cskv::bf16>(cskv::AttnArgs)", 256, 512, 1, 60000, 68000),
            ("void at::native::vectorized_elementwise_kernel<4>(int)", 128, 4, 1, 0, 900)]
    with open(p, "w") as f:
        f.write("Kernel_Name,Grid_Size_X,Grid_Size_Y,Grid_Size_Z,Start_Timestamp,End_Timestamp\n")
        for n, x, y, z, a, b in rows:
            f.write(f'"{n}",{x},{y},{z},{a},{b}\n')
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--kernel-table", str(p)],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr
    lines = [ln for ln in r.stdout.splitlines() if ln.startswith("| `")]
    assert len(lines) == 2
    assert lines[0].startswith("| `attn_mfma<512, 4, 1, -1, 1>` | 36864 | decode CSA attention (18 splits) | 2 | 23.5 | 23.0 | 24.0 |")
    assert lines[1].startswith("| `attn_merge<bf16>` | 131072 | decode split merge | 1 | 8.0 |")
