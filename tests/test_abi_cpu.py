"""C-ABI checks that need no GPU: the library loads, exports every function the
header declares, and rejects bad arguments with the documented status before
any HIP call (so these calls never touch a device)."""
import ctypes
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "cskv.h")
LIB = os.path.join(ROOT, "compressed_sparse_kv_02_amd", "libcskv.so")

OK, INVALID, SHAPE, DTYPE, MISALIGNED, WS, UNSUPPORTED = 0, -1, -2, -3, -4, -5, -6

pytestmark = pytest.mark.skipif(not os.path.exists(LIB), reason="libcskv.so not built (run __graft_entry__.build())")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:int|size_t|const char\*)\s+(\w+)\s*\(", text, flags=re.M)))


@pytest.fixture(scope="module")
def L():
    from compressed_sparse_kv_02_amd import binding
    return binding.lib()


def test_exports_every_declared_function(L):
    names = declared_functions()
    assert len(names) == 31, names
    for n in names:
        assert hasattr(L, n), n
    from compressed_sparse_kv_02_amd import binding
    assert sorted(binding.EXPORTS) == names


def test_exports_nothing_else():
    nm = shutil.which("nm")
    if nm is None:
        pytest.skip("nm not available")
    out = subprocess.run([nm, "-D", "--defined-only", LIB], capture_output=True, text=True, check=True).stdout
    exported = sorted(ln.split()[-1] for ln in out.splitlines() if ln.split()[1:2] == ["T"])
    assert exported == declared_functions()


def test_version_and_status_strings(L):
    assert L.cskv_version() == 200
    for code in range(-7, 1):
        assert len(L.cskv_status_string(code)) >= 2
    assert L.cskv_status_string(-99) == b"unknown status"


P = 0x1000  # an aligned fake device address: never dereferenced, validation fails first


def test_csa_compress_validation(L):
    f = L.csa_compress
    base = dict(Ca=P, Cb=P, Za=P, Zb=P, B=P, pCb=None, pZb=None, batch=1, T=16, c=64, m=4, pos0=0,
                norm=1, nw=None, eps=1e-6, rd=16, rb=10000.0, out=P, ld=0, dt=0, st=None)

    def call(**kw):
        a = dict(base, **kw)
        return f(*a.values())
    assert call(dt=7) == DTYPE
    assert call(c=60) == SHAPE            # c % 8
    assert call(m=0) == SHAPE
    assert call(pos0=6) == SHAPE          # pos0 % m
    assert call(rd=15) == SHAPE           # odd rope dims
    assert call(rd=128) == SHAPE          # rope dims > c
    assert call(m=256) == UNSUPPORTED
    assert call(Ca=None) == INVALID
    assert call(pCb=P) == INVALID         # prev_Cb without prev_Zb
    assert call(Ca=P + 4) == MISALIGNED
    assert call(ld=3) == SHAPE            # out_ld < T/m
    assert call(eps=0.0) == INVALID
    assert call(T=3) == OK                # no complete block: nothing to do, no launch
    assert call(batch=0) == OK


def test_hca_compress_validation(L):
    f = L.hca_compress
    base = dict(C=P, Z=None, B=None, batch=2, T=256, c=512, m=128, pos0=0, norm=1, nw=None, eps=1e-6,
                rd=64, rb=10000.0, out=P, ld=0, dt=0, st=None)

    def call(**kw):
        a = dict(base, **kw)
        return f(*a.values())
    assert call(m=5000) == UNSUPPORTED
    assert call(C=None) == INVALID
    assert call(out=None) == INVALID
    assert call(pos0=64) == SHAPE
    assert call(c=2048) == SHAPE
    assert call(T=100) == OK


def test_indexer_topk_validation(L):
    f = L.indexer_topk
    base = dict(qI=P, wI=P, KI=P, batch=1, Tq=64, N=1000, HI=64, dI=128, pos0=0, m=4, k=1024, out=P,
                ws=P, wsb=1 << 40, dt=0, st=None)

    def call(**kw):
        a = dict(base, **kw)
        return f(*a.values())
    assert call(k=4096) == UNSUPPORTED
    assert call(k=0) == SHAPE
    assert call(dI=100) == SHAPE
    assert call(dI=256) == UNSUPPORTED    # bf16 indexer supports dI 32/64/128
    assert call(HI=0) == SHAPE
    assert call(qI=None) == INVALID
    assert call(ws=None) == WS
    assert call(wsb=16) == WS
    assert call(out=P + 8) == MISALIGNED
    assert call(Tq=0) == OK
    need = L.cskv_indexer_workspace_size(1, 64, 1000, 64, 1024, 0)
    assert need >= 64 * 1000 * 4


def test_indexer_scores_validation(L):
    f = L.indexer_scores
    base = dict(qI=P, wI=P, KI=P, batch=1, Tq=64, N=1000, HI=64, dI=128, pos0=0, m=4, scores=P, ld=1024,
                bm=None, bm_ld=0, dt=0, st=None)

    def call(**kw):
        a = dict(base, **kw)
        return f(*a.values())
    assert call(ld=999) == SHAPE       # ld < N
    assert call(ld=1026) == SHAPE      # ld % 4 != 0
    assert call(scores=None) == INVALID
    assert call(scores=P + 4) == MISALIGNED
    # block maxima: one per 32 entries (ceil(1000 / 32) = 32), bf16 scorers only
    assert call(bm=P, bm_ld=32, dt=1) == UNSUPPORTED
    assert call(bm=P, bm_ld=28) == SHAPE
    assert call(bm=P, bm_ld=34) == SHAPE
    assert call(bm=P + 8, bm_ld=32) == MISALIGNED
    assert call(bm=P, bm_ld=32, Tq=0) == OK
    assert call(Tq=0) == OK


def test_topk_select_validation(L):
    f = L.topk_select
    base = dict(scores=P, ld=1024, bm=None, bm_ld=0, batch=1, Tq=4, N=1000, pos0=0, m=4, k=64, out=P, ws=None,
                wsb=0, st=None)

    def call(**kw):
        a = dict(base, **kw)
        return f(*a.values())
    assert call(k=4096) == UNSUPPORTED
    assert call(k=0) == SHAPE
    assert call(ld=999) == SHAPE       # ld < N
    assert call(ld=1002) == SHAPE      # ld % 4 != 0
    assert call(out=None) == INVALID
    assert call(out=P + 8) == MISALIGNED
    assert call(ws=P + 8, wsb=1 << 20) == MISALIGNED
    assert call(bm=P, bm_ld=28) == SHAPE     # fewer than ceil(N / 32) blocks per row
    assert call(bm=P, bm_ld=33) == SHAPE     # bm_ld % 4 != 0
    assert call(bm=P + 4, bm_ld=32) == MISALIGNED
    assert call(Tq=0) == OK
    # the two-kernel route is offered to few rows of at least 4 x 8192 entries only
    assert L.cskv_topk_workspace_size(8, 1, 262144, 1024) > 0
    assert L.cskv_topk_workspace_size(8, 1, 20000, 1024) == 0
    assert L.cskv_topk_workspace_size(2, 4096, 262144, 1024) == 0
    assert L.cskv_topk_workspace_size(1, 1, 1 << 21, 1024) == 0   # more than 128 parts


def test_fp8_indexer_validation(L):
    q = L.cskv_quantize_fp8
    assert q(P, 10, 128, 2, P, P, None) == DTYPE     # input must be bf16 or fp32
    assert q(P, 10, 130, 0, P, P, None) == SHAPE     # dim % 4
    assert q(P, 10, 2048, 0, P, P, None) == SHAPE    # dim > 1024
    assert q(P, 10, 128, 0, None, P, None) == INVALID
    assert q(P, 10, 128, 0, P + 4, P, None) == MISALIGNED
    assert q(P, 0, 128, 0, P, P, None) == OK
    s = L.indexer_scores_fp8
    base = dict(q=P, qs=P, w=P, k=P, ks=P, batch=1, Tq=4, N=1000, HI=64, dI=128, pos0=0, m=4, sc=P, ld=1024,
                st=None)

    def call(**kw):
        a = dict(base, **kw)
        return s(*a.values())
    assert call(dI=96) == UNSUPPORTED
    assert call(HI=0) == SHAPE
    assert call(ld=999) == SHAPE
    assert call(qs=None) == INVALID
    assert call(ks=P + 4) == MISALIGNED
    assert call(Tq=0) == OK
    t = L.indexer_topk_fp8
    tb = dict(q=P, qs=P, w=P, k=P, ks=P, batch=1, Tq=64, N=1000, HI=64, dI=128, pos0=0, m=4, kk=1024, out=P,
              ws=P, wsb=1 << 40, st=None)

    def tcall(**kw):
        a = dict(tb, **kw)
        return t(*a.values())
    assert tcall(kk=4096) == UNSUPPORTED
    assert tcall(ws=None) == WS
    assert tcall(dI=32) == UNSUPPORTED
    assert L.cskv_indexer_workspace_size(1, 64, 1000, 64, 1024, 2) >= 64 * 1000 * 4
    # FP4 entry points share the validation
    assert L.cskv_quantize_fp4(P, 10, 130, 0, P, P, None) == SHAPE
    assert L.cskv_quantize_fp4(P, 10, 128, 2, P, P, None) == DTYPE
    a = dict(base)
    a.update(dI=96)
    assert L.indexer_scores_fp4(*a.values()) == UNSUPPORTED
    a = dict(tb)
    a.update(ws=None)
    assert L.indexer_topk_fp4(*a.values()) == WS
    assert L.cskv_indexer_workspace_size(1, 64, 1000, 64, 1024, 3) >= 64 * 1000 * 4


def test_mx_indexer_validation(L):
    for fmt in ("mxfp4", "mxfp8"):
        q = getattr(L, f"cskv_quantize_{fmt}")
        assert q(P, 10, 128, 2, P, P, None) == DTYPE     # input must be bf16 or fp32
        assert q(P, 10, 48, 0, P, P, None) == SHAPE      # dim % 32 (one scale per 32 values)
        assert q(P, 10, 2048, 0, P, P, None) == SHAPE    # dim > 1024
        assert q(P, 10, 128, 0, P, None, None) == INVALID
        assert q(P, 10, 128, 0, P, P + 4, None) == MISALIGNED
        assert q(P, 0, 128, 0, P, P, None) == OK
        s = getattr(L, f"indexer_scores_{fmt}")
        base = dict(q=P, qs=P, w=P, k=P, ks=P, batch=1, Tq=4, N=1000, HI=64, dI=128, pos0=0, m=4, sc=P, ld=1024,
                    st=None)
        for kw, want in ((dict(dI=64), UNSUPPORTED),   # 4 scale bytes per row: dI = 128 only
                         (dict(HI=0), SHAPE), (dict(ld=999), SHAPE), (dict(qs=None), INVALID),
                         (dict(ks=P + 4), MISALIGNED), (dict(Tq=0), OK)):
            assert s(*dict(base, **kw).values()) == want, (fmt, kw)
        t = getattr(L, f"indexer_topk_{fmt}")
        tb = dict(q=P, qs=P, w=P, k=P, ks=P, batch=1, Tq=64, N=1000, HI=64, dI=128, pos0=0, m=4, kk=1024, out=P,
                  ws=P, wsb=1 << 40, st=None)
        for kw, want in ((dict(kk=4096), UNSUPPORTED), (dict(ws=None), WS), (dict(dI=64), UNSUPPORTED)):
            assert t(*dict(tb, **kw).values()) == want, (fmt, kw)
    assert L.cskv_indexer_workspace_size(1, 64, 1000, 64, 1024, 4) >= 64 * 1000 * 4
    assert L.cskv_indexer_workspace_size(1, 64, 1000, 64, 1024, 5) >= 64 * 1000 * 4


def test_kv8_validation(L):
    q = L.cskv_quantize_kv_fp8
    assert q(P, 1, 4, 512, 64, 2, P, P, 0, None) == DTYPE
    assert q(P, 1, 4, 512, 60, 0, P, P, 0, None) == SHAPE     # rope dims not a multiple of 8
    assert q(P, 1, 4, 520, 64, 0, P, P, 0, None) == SHAPE     # non-RoPE dims not a multiple of 16
    assert q(P, 1, 4, 512, 64, 0, P, P, 3, None) == SHAPE     # out_ld < n
    assert q(P, 1, 4, 512, 64, 0, None, P, 0, None) == INVALID
    assert q(P, 1, 0, 512, 64, 0, P, P, 0, None) == OK
    f = L.compressed_attn_prefill_kv8
    base = dict(mode=0, q=P, kv=P, ks=P, idx=P, win=P, wp0=0, W=64, sink=None, batch=1, Tq=64, N=16,
                pos0=0, m=4, k=16, w=16, H=64, d=512, qn=1, qnw=None, eps=1e-6, rd=64, rb=1e4,
                scale=0.0, roo=1, ws=None, wsb=0, out=P, lse=None, st=None)

    def call(**kw):
        a = dict(base, **kw)
        return f(*a.values())
    assert call(ks=None) == INVALID
    assert call(rd=60) == SHAPE
    assert call(rd=48) == UNSUPPORTED
    assert call(ks=P + 4) == MISALIGNED
    assert call(Tq=0) == OK
    # HCA with a workspace: the entries are widened into it first, so it is checked before any launch
    sz = L.cskv_prefill_kv8_workspace_size
    assert sz(1, 2, 16, 512) == 2 * 16 * 512 * 2 and sz(0, 2, 16, 512) == 0 and sz(1, 0, 16, 512) == 0
    need = sz(1, 1, 16, 512)
    assert call(mode=1, ws=P, wsb=need - 1) == WS
    assert call(mode=1, ws=P + 8, wsb=need) == MISALIGNED
    assert call(mode=1, ws=P, wsb=need, rd=48) == UNSUPPORTED
    assert call(mode=0, ws=P, wsb=0, Tq=0) == OK  # CSA ignores the workspace


def test_attention_validation(L):
    for fname in ("compressed_attn_prefill", "compressed_attn_decode"):
        f = getattr(L, fname)
        base = dict(mode=0, q=P, kv=P, idx=P, win=P, wp0=0, W=64, sink=None, batch=1, Tq=64, N=16,
                    pos0=0, m=4, k=16, w=16, H=64, d=512, qn=1, qnw=None, eps=1e-6, rd=64, rb=1e4,
                    scale=0.0, roo=1)
        extra = dict(ns=0, ws=P, wsb=1 << 40) if fname.endswith("decode") else {}
        tail = dict(out=P, lse=None, dt=0, st=None)

        def call(**kw):
            a = dict(base, **extra, **tail)
            a.update(kw)
            return f(*a.values())
        assert call(mode=3) == INVALID
        assert call(dt=2) == DTYPE
        assert call(d=96) == UNSUPPORTED    # bf16 head dims 64/128/256/512
        assert call(H=0) == SHAPE
        assert call(w=0) == SHAPE
        assert call(k=0) == SHAPE
        assert call(k=4096) == UNSUPPORTED
        assert call(W=63) == SHAPE           # window rows do not reach the last query
        assert call(wp0=-1) == SHAPE         # window base before position 0
        assert call(idx=None) == INVALID     # CSA needs indices
        assert call(q=P + 2) == MISALIGNED
        assert call(Tq=0) == OK
        if fname.endswith("decode"):
            assert call(ns=300) == SHAPE


def test_projection_validation(L):
    f = L.cskv_lowrank_proj
    assert f(P, P, P, 64, 256, 8192, 1, None) == DTYPE        # bf16 only
    assert f(P, P, P, 64, 96, 8192, 0, None) == SHAPE         # r not a multiple of 64
    assert f(P, P, P, 64, 256, 8190, 0, None) == SHAPE        # n_out not a multiple of 8
    assert f(P, P, P, -1, 256, 8192, 0, None) == SHAPE
    assert f(None, P, P, 64, 256, 8192, 0, None) == INVALID
    assert f(P, P + 8, P, 64, 256, 8192, 0, None) == MISALIGNED
    assert f(P, P, P, 0, 256, 8192, 0, None) == OK            # no tokens: nothing launched
    g = L.cskv_grouped_out_proj
    base = dict(o=P, Wg=P, Wo=P, mid=P, y=P, T=64, H=64, d=512, G=8, dg=1024, D=4096, dt=0, st=None)

    def call(**kw):
        a = dict(base, **kw)
        return g(*a.values())
    assert call(dt=1) == DTYPE
    assert call(G=7) == SHAPE       # H not a multiple of G
    assert call(d=32, H=8, G=8) == SHAPE   # (H/G) d = 32 not a multiple of 64
    assert call(dg=1020) == SHAPE
    assert call(D=4100) == SHAPE
    assert call(mid=None) == INVALID
    assert call(y=P + 2) == MISALIGNED
    assert call(T=0) == OK


def test_binding_refuses_cpu_tensors():
    import torch
    from compressed_sparse_kv_02_amd import binding
    x = torch.zeros(1, 8, 64)
    with pytest.raises(binding.CskvError):
        binding.hca_compress(x, m=1)


def test_binding_rejects_appends_past_the_cache():
    # the extent checks run before any device access, so CPU tensors reach them
    import torch
    from compressed_sparse_kv_02_amd import binding
    x = torch.zeros(2, 16, 64)
    B = torch.zeros(8, 64)
    cache = torch.zeros(2, 10, 64)
    for row0 in (-1, 7, 10):                       # 16 / 4 = 4 new rows: rows 7..10 overflow a 10-row cache
        with pytest.raises(binding.CskvError, match="do not fit"):
            binding.csa_compress(x, x, x, x, B, 4, out=cache, out_row0=row0)
    with pytest.raises(binding.CskvError, match="do not fit"):
        binding.hca_compress(x, None, None, 4, out=cache, out_row0=7)
    with pytest.raises(binding.CskvError, match="out must be"):
        binding.hca_compress(x, None, None, 4, out=torch.zeros(1, 10, 64))   # wrong batch
    with pytest.raises(binding.CskvError, match="dtype"):
        binding.hca_compress(x, None, None, 4, out=torch.zeros(2, 10, 64, dtype=torch.bfloat16))
    with pytest.raises(binding.CskvError, match="without scales"):
        binding.quantize_kv_fp8(torch.zeros(2, 4, 64), 16, out=torch.zeros(2, 10, 80, dtype=torch.uint8))
    with pytest.raises(binding.CskvError, match="do not fit"):
        binding.quantize_kv_fp8(torch.zeros(2, 4, 64), 16, out=torch.zeros(2, 10, 80, dtype=torch.uint8),
                                scales=torch.zeros(2, 10), out_row0=8)
    # in range: the device check is what fails on the CPU
    with pytest.raises(binding.CskvError, match="not on the GPU"):
        binding.csa_compress(x, x, x, x, B, 4, out=cache, out_row0=6)


def test_binding_rejects_mismatched_attention_buffers():
    # entry rows, FP8 scales, sinks and norm weights bound what the kernels read: checked first
    import torch
    from compressed_sparse_kv_02_amd import binding
    bt, Tq, H, d, N = 2, 4, 8, 64, 12
    q = torch.zeros(bt, Tq, H, d)
    win = torch.zeros(bt, 16, d)
    kv = torch.zeros(bt, N, d)
    call = lambda **kw: binding.compressed_attn_prefill(binding.HCA, q, kw.pop("kv", kv), None, win, 0,
                                                        kw.pop("sink", None), 0, 4, 16, **kw)
    with pytest.raises(binding.CskvError, match="kv must be"):
        call(kv=torch.zeros(bt, N, d + 8))
    with pytest.raises(binding.CskvError, match="kv must be"):
        call(kv=torch.zeros(bt, N, d, dtype=torch.bfloat16))
    with pytest.raises(binding.CskvError, match="sink"):
        call(sink=torch.zeros(H + 1))
    with pytest.raises(binding.CskvError, match="q_norm_w"):
        call(q_norm_w=torch.zeros(d - 1))
    rb = binding.kv_fp8_row_bytes(d, 16)
    kv8 = torch.zeros(bt, N, rb, dtype=torch.uint8)
    with pytest.raises(binding.CskvError, match="kv must be uint8"):
        call(kv=torch.zeros(bt, N, rb + 16, dtype=torch.uint8), kv_scale=torch.zeros(bt, N), rope_dims=16)
    with pytest.raises(binding.CskvError, match="kv_scale"):
        call(kv=kv8, kv_scale=torch.zeros(bt, N - 1), rope_dims=16)
    with pytest.raises(binding.CskvError, match="not on the GPU"):  # consistent buffers reach the device check
        call()


def test_decode_workspace_size_follows_the_split_policy(L):
    f = L.cskv_decode_workspace_size
    per = lambda b, tq, s, H=64, d=512: b * tq * s * H * (d + 2) * 4
    # automatic splits: at most ceil(256 / (batch * Tq)), nothing when that is one split
    assert f(8, 1, 64, 512, 0) == per(8, 1, 32)
    assert f(1, 1, 64, 512, 0) == per(1, 1, 256)
    assert f(3, 1, 64, 512, 0) == per(3, 1, 86)
    assert f(2, 4096, 64, 512, 0) == 0 and f(256, 1, 64, 512, 0) == 0
    assert f(8, 1, 64, 512, 1) == 0
    assert f(8, 1, 64, 512, 7) == per(8, 1, 7)
    # arguments the call rejects size to 0
    assert f(8, 1, 64, 512, 257) == 0 and f(8, 1, 64, 512, -1) == 0 and f(0, 1, 64, 512, 0) == 0
    # a decode call with too small a workspace fails validation before any launch
    a = dict(mode=1, q=P, kv=P, idx=None, win=P, wp0=0, W=128, sink=None, batch=8, Tq=1, N=8192,
             pos0=1 << 20, m=128, k=0, w=128, H=64, d=512, qn=1, qnw=None, eps=1e-6, rd=64, rb=1e4,
             sc=0.0, ro=1, ns=0, ws=P, wsb=f(8, 1, 64, 512, 0) - 1, out=P, lse=None, dt=0, st=None)
    assert L.compressed_attn_decode(*a.values()) == WS


def test_decode_noalloc_rejects_explicit_splits_beyond_its_scratch(L):
    from compressed_sparse_kv_02_amd import binding
    f = L.compressed_attn_decode_noalloc
    a = dict(mode=1, q=P, kv=P, idx=None, win=P, wp0=0, W=128, sink=None, batch=8, Tq=1, N=8192,
             pos0=1 << 20, m=128, k=0, w=128, H=64, d=512, qn=1, qnw=None, eps=1e-6, rd=64, rb=1e4,
             sc=0.0, ro=1, ns=256, out=P, lse=None, dt=0, st=None)
    # 8 x 256 splits x 64 heads x 514 x 4 bytes = 269 MB of partials > 64 MiB: refused before any HIP call
    assert 8 * 256 * 64 * 514 * 4 > binding.NOALLOC_SCRATCH_BYTES
    assert f(*a.values()) == WS
    assert f(*dict(a, ns=257).values()) == SHAPE
    assert f(*dict(a, dt=5).values()) == DTYPE
    assert f(*dict(a, out=None).values()) == INVALID
    assert f(*dict(a, q=P + 8).values()) == MISALIGNED
    # the binding refuses to allocate an output for it
    import torch
    with pytest.raises(binding.CskvError, match="out must be given"):
        binding.compressed_attn_decode_noalloc(1, torch.zeros(1, 1, 4, 64), torch.zeros(1, 8, 64), None,
                                               torch.zeros(1, 4, 64), 0, None, 3, 1, 4, out=None)
