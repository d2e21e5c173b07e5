"""GPU parity: the HIP path (through the C ABI) against the CPU oracle on the
same seeded inputs. Stage tests feed both sides generator-made inputs for
every stage; end-to-end tests run the whole layer on both sides."""
import dataclasses
import math
import warnings

import numpy as np
import pytest
import torch

from oracle import cskv_oracle as O
from compressed_sparse_kv_02_amd import binding as B
from compressed_sparse_kv_02_amd import layer as LY
from compressed_sparse_kv_02_amd.synth import normal_device, uniform_device
from tests.parity_utils import (assert_storage_close, check_topk_row, check_topk_row_bounded, fp8_refined_bound,
                                fp8_score_bound, mxfp4_score_bound, mxfp8_refined_bound, mxfp8_score_bound,
                                key_rounding_band, np64, oracle_layer, ParityCount)

pytestmark = pytest.mark.gpu
DEV = "cuda"
TD = {"bf16": torch.bfloat16, "f32": torch.float32}
ATOL = {"bf16": 2e-2, "f32": 1e-4}


def say(*a):
    print(*a, flush=True)


def gen(seed, name, shape, dtype="bf16", std=1.0):
    return normal_device(seed, name, shape, std, dtype, DEV)


# ----------------------------------------------------------------------------- compressors

@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("c,m,T,pos0,norm,rope", [
    (64, 4, 203, 0, True, 16), (512, 4, 1000, 0, True, 64), (128, 4, 77, 96, False, 0),
    (512, 4, 64, 4096, True, 64), (32 * 8, 2, 9, 0, True, 8), (64, 1, 33, 0, False, 0),
    (96, 4, 130, 8, True, 6), (512, 20, 100, 40, True, 64)])
def test_csa_compress(dtype, c, m, T, pos0, norm, rope):
    say("csa_compress", dtype, c, m, T, pos0, norm, rope)
    bt = 2
    g = lambda nm, sh: gen(11, f"cc.{nm}", sh, dtype)
    Ca, Cb, Za, Zb = (g(nm, (bt, T, c)) for nm in ("Ca", "Cb", "Za", "Zb"))
    Bb = g("B", (2 * m, c))
    prev = (g("pCb", (bt, m, c)), g("pZb", (bt, m, c))) if pos0 else (None, None)
    out = B.csa_compress(Ca, Cb, Za, Zb, Bb, m, pos0, *prev, apply_norm=norm, rope_dims=rope)
    torch.cuda.synchronize()
    assert out.shape == (bt, T // m, c)
    for b in range(bt):
        ref = O.csa_compress(np64(Ca[b]), np64(Cb[b]), np64(Za[b]), np64(Zb[b]), np64(Bb), m, pos0,
                             np64(prev[0][b]) if pos0 else None, np64(prev[1][b]) if pos0 else None,
                             apply_norm=norm, rope_dims=rope)
        assert_storage_close(np64(out[b]), ref, dtype, f"csa b={b}")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("c,m,T,pos0,withZ,norm,rope", [
    (512, 128, 300, 0, True, True, 64), (512, 128, 1024, 128 * 7, True, True, 64), (64, 16, 50, 0, False, True, 16),
    (512, 1, 37, 1000, False, True, 64), (128, 1, 5, 0, True, False, 0), (512, 4096, 4096, 0, True, True, 64),
    (1024, 1, 9, 3, False, True, 10), (1024, 64, 200, 128, True, True, 64), (40, 8, 100, 16, True, True, 2),
    (512, 128, 260, 256, False, True, 64), (256, 48, 100, 0, False, False, 0)])
def test_hca_compress(dtype, c, m, T, pos0, withZ, norm, rope):
    say("hca_compress", dtype, c, m, T, pos0, withZ, norm, rope)
    bt = 2
    C = gen(12, "hc.C", (bt, T, c), dtype)
    Z = gen(12, "hc.Z", (bt, T, c), dtype) if withZ else None
    Bb = gen(12, "hc.B", (m, c), dtype, 0.1) if withZ else None
    out = B.hca_compress(C, Z, Bb, m, pos0, apply_norm=norm, rope_dims=rope)
    torch.cuda.synchronize()
    for b in range(bt):
        ref = O.hca_compress(np64(C[b]), np64(Z[b]) if withZ else None, np64(Bb) if withZ else None, m, pos0,
                             apply_norm=norm, rope_dims=rope)
        assert_storage_close(np64(out[b]), ref, dtype, f"hca b={b}")


def test_compress_append_in_place():
    say("compress append in place")
    c, m, T = 128, 4, 64
    Ca, Cb, Za, Zb = (gen(13, f"ap.{n}", (2, T, c)) for n in ("Ca", "Cb", "Za", "Zb"))
    Bb = gen(13, "ap.B", (2 * m, c))
    cache = torch.full((2, 40, c), 7.0, dtype=torch.bfloat16, device=DEV)
    B.csa_compress(Ca, Cb, Za, Zb, Bb, m, out=cache, out_row0=20)
    ref = B.csa_compress(Ca, Cb, Za, Zb, Bb, m)
    torch.cuda.synchronize()
    assert torch.equal(cache[:, 20:36], ref)
    assert (cache[:, :20] == 7).all() and (cache[:, 36:] == 7).all()


# ----------------------------------------------------------------------------- indexer + top-k

def _indexer_case(dtype, bt, Tq, N, HI, dI, pos0, m, k, seed, integer=False):
    if integer:  # small integers: exact scores, many exact ties
        g = torch.Generator(device=DEV).manual_seed(seed)
        qI = torch.randint(-2, 3, (bt, Tq, HI, dI), generator=g, device=DEV).to(TD[dtype])
        KI = torch.randint(-2, 3, (bt, N, dI), generator=g, device=DEV).to(TD[dtype])
        wI = torch.randint(0, 3, (bt, Tq, HI), generator=g, device=DEV).float()
    else:
        qI = gen(seed, "ix.q", (bt, Tq, HI, dI), dtype)
        KI = gen(seed, "ix.k", (bt, N, dI), dtype)
        wI = uniform_device(seed, "ix.w", (bt, Tq, HI), DEV)
    idx = B.indexer_topk(qI, wI, KI, pos0, m, k)
    torch.cuda.synchronize()
    return qI, wI, KI, idx


@pytest.mark.parametrize("dtype,bt,Tq,N,HI,dI,pos0,m,k", [
    ("f32", 1, 512, 128, 2, 32, 0, 4, 16),          # tiny CSA indexer shape
    ("bf16", 2, 300, 400, 64, 128, 0, 4, 64),       # ragged rows, V_t both below and above k
    ("bf16", 1, 77, 5000, 20, 64, 16000, 4, 100),   # chunk on a cache, HI not a multiple of 32
    ("bf16", 3, 5, 70000, 64, 128, 4 * 70000, 4, 1024),  # few queries, long rows (key splits)
    ("bf16", 1, 130, 3000, 32, 32, 3000 * 4 - 64, 4, 2048),  # max k
])
def test_indexer_topk(dtype, bt, Tq, N, HI, dI, pos0, m, k):
    say("indexer_topk", dtype, bt, Tq, N, HI, dI, pos0, m, k)
    qI, wI, KI, idx = _indexer_case(dtype, bt, Tq, N, HI, dI, pos0, m, k, seed=21)
    idx = idx.cpu().numpy()
    rows = range(Tq) if Tq <= 80 else sorted(set(np.linspace(0, Tq - 1, 60).astype(int)) | {0, Tq - 1})
    n_band = 0
    for b in range(bt):
        K = np64(KI[b])
        for r in rows:
            I = O.indexer_scores(np64(qI[b, r:r + 1]), np64(wI[b, r:r + 1]), K, pos0 + r, m)[0]
            n_band += check_topk_row(idx[b, r], I, O.visible(pos0 + r, m, N), k, what=f"b{b} r{r}")
    say("  tie-band differences:", n_band)


def test_indexer_topk_exact_ties():
    say("indexer_topk integer ties")
    bt, Tq, N, HI, dI, k = 2, 64, 600, 32, 32, 50
    qI, wI, KI, idx = _indexer_case("bf16", bt, Tq, N, HI, dI, 4 * 500, 4, k, seed=5, integer=True)
    idx = idx.cpu().numpy()
    for b in range(bt):
        K = np64(KI[b])
        for r in range(Tq):
            I = O.indexer_scores(np64(qI[b, r:r + 1]), np64(wI[b, r:r + 1]), K, 2000 + r, 4)[0]
            V = O.visible(2000 + r, 4, N)
            # integer scores are exact in fp32: the selection must equal the oracle's, ties included
            assert np.array_equal(idx[b, r], O.topk_row(I, V, k)), (b, r)


def test_indexer_decode_1m_full():
    say("indexer_topk decode 1M: batch 8, 262144 keys")
    qI, wI, KI, idx = _indexer_case("bf16", 8, 1, 262144, 64, 128, 1 << 20, 4, 1024, seed=4)
    idx = idx.cpu().numpy()
    for b in range(8):
        I = O.indexer_scores(np64(qI[b]), np64(wI[b]), np64(KI[b]), 1 << 20, 4)[0]
        check_topk_row(idx[b, 0], I, 262144, 1024, what=f"b{b}")


def block_max_of(sc, pos0, m, N):
    """[batch, Tq, ceil(N/32)] int64: each 32-entry block's largest order key among the first V_t
    scores of a row (key: the fp32 bits with the sign bit set for non-negative scores, all bits
    flipped for negative ones; 0 where the block holds no visible entry)."""
    bt, Tq, _ = sc.shape
    nb = (N + 31) // 32
    u = sc[..., :N].contiguous().view(torch.int32).to(torch.int64) & 0xFFFFFFFF
    key = torch.where(u >= 0x80000000, u ^ 0xFFFFFFFF, u | 0x80000000)
    V = torch.tensor([O.visible(pos0 + r, m, N) for r in range(Tq)], device=sc.device)
    s = torch.arange(N, device=sc.device)
    key = torch.where(s[None, None, :] < V[None, :, None], key, torch.zeros_like(key))
    return torch.nn.functional.pad(key, (0, nb * 32 - N)).view(bt, Tq, nb, 32).amax(-1)


def _as_block_max(key, N):
    """int64 keys -> the int32 bit patterns of a [batch, Tq, block_max_ld(N)] block-maximum matrix."""
    bm = torch.zeros(*key.shape[:2], B.block_max_ld(N), dtype=torch.int32, device=key.device)
    bm[..., :key.shape[-1]] = torch.where(key >= 2 ** 31, key - 2 ** 32, key).to(torch.int32)
    return bm


@pytest.mark.parametrize("bt,Tq,N,HI,dI,pos0,k", [
    (3, 1, 90000, 64, 128, 4 * 90000, 1024),          # decode rows of 2813 blocks
    (2, 5, 262144, 64, 128, 4 * 262144 - 5, 1024),    # 8192 blocks (the most)
    (1, 63, 5000, 20, 64, 4 * 5000 - 70, 64),         # the most queries written, 20 heads, 157 blocks
    (2, 3, 40000, 64, 128, 4 * 40000, 1024),          # 1250 blocks, fewer than 2k: maxima unused
    (2, 100, 70000, 64, 128, 4 * 70000 - 120, 1024),  # 100 queries: maxima left untouched, unused
])
def test_indexer_block_max(bt, Tq, N, HI, dI, pos0, k):
    """indexer_scores' block maxima (calls of fewer than 64 queries) equal the definition over the
    scores it wrote; the selection given them equals the selection without them, indexer_topk's,
    and (sampled rows) the oracle's."""
    say("indexer block maxima", bt, Tq, N, HI, dI, pos0, k)
    qI = gen(29, "bm.q", (bt, Tq, HI, dI))
    KI = gen(29, "bm.k", (bt, N, dI))
    wI = uniform_device(29, "bm.w", (bt, Tq, HI), DEV)
    bm = torch.full((bt, Tq, B.block_max_ld(N)), -1, dtype=torch.int32, device=DEV)
    sc = B.indexer_scores(qI, wI, KI, pos0, 4, block_max=bm)
    a = B.topk_select(sc, N, pos0, 4, k, block_max=bm)
    b = B.topk_select(sc, N, pos0, 4, k)
    c = B.indexer_topk(qI, wI, KI, pos0, 4, k)
    torch.cuda.synchronize()
    if Tq < 64:
        key = block_max_of(sc, pos0, 4, N).cpu()
        got = bm.cpu().to(torch.int64) & 0xFFFFFFFF
        for r in range(Tq):
            nb = (O.visible(pos0 + r, 4, N) + 31) // 32
            assert torch.equal(got[:, r, :nb], key[:, r, :nb]), r
    else:
        assert bool((bm == -1).all())
    assert torch.equal(a, b)
    assert torch.equal(a, c)
    a = a.cpu().numpy()
    for bb, r in {(0, 0), (bt - 1, Tq - 1)}:
        I = O.indexer_scores(np64(qI[bb, r:r + 1]), np64(wI[bb, r:r + 1]), np64(KI[bb]), pos0 + r, 4)[0]
        check_topk_row(a[bb, r], I, O.visible(pos0 + r, 4, N), k, what=f"b{bb} r{r}")


@pytest.mark.parametrize("kind,bt,Tq,N,k", [
    ("normal", 2, 3, 200000, 1024),
    ("normal", 1, 2, 262144, 2048),   # max k: 32 parts x 256 candidates
    ("ramp", 1, 2, 100000, 1024),     # the top-k sits in the last part: fallback route
    ("descending", 1, 1, 100000, 1024),  # the top-k sits in the first part: fallback route
    ("ties", 2, 2, 65536, 2048),      # 16 distinct values: ties across parts
    ("equal", 1, 1, 40000, 100),      # one value: the first k indices
    ("normal", 8, 1, 262144, 1024),   # the decode shape: block maxima, 8192 blocks per row
    ("normal", 1, 2, 40000, 1024),    # 1250 blocks, fewer than 2k: parts + merge
    ("normal", 1, 2, 300000, 1024),   # more than 8192 blocks: parts + merge
    ("ties", 1, 2, 262144, 1024),     # block maxima route, candidates overflow LDS: exact fallback
])
def test_topk_split_route(kind, bt, Tq, N, k):
    """Few long rows go through a several-workgroups-per-row route (block maxima from 2k up to 8192
    blocks of 32 entries, parts + merge otherwise); it must equal the one-workgroup-per-row route, the
    selection given block maxima, and the oracle's top-k exactly (same fp32 scores on every side)."""
    say("topk split route", kind, bt, Tq, N, k)
    ld = B.score_ld(N)
    if kind == "normal":
        sc = normal_device(61, "tk.normal", (bt, Tq, ld), 1.0, "f32", DEV)
    elif kind == "ties":
        sc = torch.floor(uniform_device(61, "tk.ties", (bt, Tq, ld), DEV) * 16.0)
    elif kind == "equal":
        sc = torch.full((bt, Tq, ld), 0.5, dtype=torch.float32, device=DEV)
    else:
        ramp = torch.arange(ld, dtype=torch.float32, device=DEV)
        sc = (ramp if kind == "ramp" else -ramp).expand(bt, Tq, ld).contiguous()
    pos0 = 4 * N - Tq + 1 - 8   # rows of V = N - 2 .. N
    assert B.topk_workspace_bytes(bt, Tq, N, k) > 0
    ws = torch.empty(B.topk_workspace_bytes(bt, Tq, N, k), dtype=torch.uint8, device=DEV)
    a = B.topk_select(sc, N, pos0, 4, k, workspace=ws)
    b = B.topk_select(sc, N, pos0, 4, k)
    c = B.topk_select(sc, N, pos0, 4, k, block_max=_as_block_max(block_max_of(sc, pos0, 4, N), N))
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    assert torch.equal(a, c)
    a, scn = a.cpu().numpy(), sc.cpu().numpy().astype(np.float64)
    for bb in range(bt):
        for r in range(Tq):
            V = O.visible(pos0 + r, 4, N)
            assert np.array_equal(a[bb, r], O.topk_row(scn[bb, r], V, k)), (bb, r)


# ----------------------------------------------------------------------------- FP8 (E4M3) indexer

@pytest.mark.parametrize("dtype,rows,dim", [("bf16", 1000, 128), ("f32", 333, 64), ("bf16", 7, 1024),
                                            ("bf16", 130, 4)])
def test_quantize_fp8(dtype, rows, dim):
    say("quantize_fp8", dtype, rows, dim)
    x = gen(71, "q8.x", (rows, dim), dtype, std=3.0)
    x[1] = 0.0                                     # a zero row
    x[2, : dim // 2] = -x[2, dim // 2: 2 * (dim // 2)]  # exact ties in magnitude
    x[3] *= 1e-30 if dtype == "f32" else 1.0       # tiny values: subnormal codes after scaling
    codes, scales = B.quantize_fp8(x)
    torch.cuda.synchronize()
    oc, osc = O.quantize_rows_fp8(np64(x).astype(np.float32))
    assert np.array_equal(codes.cpu().numpy(), oc)
    assert np.array_equal(scales.cpu().numpy(), osc)


def _fp8_case(bt, Tq, N, HI, dI, seed):
    qI = gen(seed, "i8.q", (bt, Tq, HI, dI))
    KI = gen(seed, "i8.k", (bt, N, dI))
    wI = uniform_device(seed, "i8.w", (bt, Tq, HI), DEV)
    qc, qs = B.quantize_fp8(qI)
    kc, ks = B.quantize_fp8(KI)
    torch.cuda.synchronize()
    return qI, KI, wI, qc, qs, kc, ks


@pytest.mark.parametrize("bt,Tq,N,HI,dI,pos0,m,k", [
    (2, 300, 2000, 64, 128, 4 * 2000 - 300, 4, 256),   # prefill route (8 queries per workgroup), ragged tail
    (1, 77, 5000, 20, 64, 16000, 4, 100),             # dI 64, HI not a multiple of 32
    (3, 5, 70000, 64, 128, 4 * 70000, 4, 1024),       # decode route (streaming waves), two-kernel top-k
    (1, 2, 3000, 128, 128, 3000 * 4 - 2, 4, 2048),    # 128 heads, max k
    (1, 1024, 7000, 64, 128, 4 * 7000 - 1024, 4, 512),  # spans of 3 and 4 key tiles, partial last tiles
])
def test_indexer_fp8(bt, Tq, N, HI, dI, pos0, m, k):
    """FP8 scores and top-k against the oracle on its own quantisation of the same raw inputs."""
    say("indexer fp8", bt, Tq, N, HI, dI, pos0, m, k)
    qI, KI, wI, qc, qs, kc, ks = _fp8_case(bt, Tq, N, HI, dI, seed=31)
    sc = B.indexer_scores_fp8(qc, qs, wI, kc, ks, pos0, m)
    idx = B.indexer_topk_fp8(qc, qs, wI, kc, ks, pos0, m, k)
    torch.cuda.synchronize()
    sc, idx = sc.cpu().numpy(), idx.cpu().numpy()
    rows = range(Tq) if Tq <= 80 else sorted(set(np.linspace(0, Tq - 1, 40).astype(int)) | {0, Tq - 1})
    n_band, worst, worst_ref = 0, 0.0, 0.0
    for b in range(bt):
        okc, oks = O.quantize_rows_fp8(np64(KI[b]).astype(np.float32))
        assert np.array_equal(okc, kc[b].cpu().numpy())
        for r in rows:
            oqc, oqs = O.quantize_rows_fp8(np64(qI[b, r]).astype(np.float32))
            I = O.indexer_scores_fp8(oqc[None], oqs[None], np64(wI[b, r:r + 1]), okc, oks, pos0 + r, m)[0]
            V = O.visible(pos0 + r, m, N)
            if V == 0:
                continue
            cheap = fp8_score_bound(oqc, oqs, np64(wI[b, r]), okc, oks, V)
            bound = fp8_refined_bound(oqc, oqs, np64(wI[b, r]), okc, oks, V, k, I)
            err = np.abs(sc[b, r, :V] - I[:V])
            assert (err <= bound).all(), (b, r, float((err / bound).max()))
            worst = max(worst, float((err / bound).max()))
            ref = bound < cheap
            if ref.any():
                worst_ref = max(worst_ref, float((err[ref] / bound[ref]).max()))
            n_band += check_topk_row_bounded(idx[b, r], I, bound, V, k, what=f"b{b} r{r}")
    msg = (f"fp8 {bt}x{Tq}x{N} k={k}: undecided entries {n_band}; largest error / bound {worst:.3g} "
           f"(entries bounded product by product: {worst_ref:.3g})")
    say("  " + msg)
    warnings.warn(ParityCount(msg))


def test_indexer_fp8_decode_1m():
    say("indexer fp8 decode 1M: batch 8, 262144 keys")
    N, pos0 = 262144, 1 << 20
    qI, KI, wI, qc, qs, kc, ks = _fp8_case(8, 1, N, 64, 128, seed=4)
    idx = B.indexer_topk_fp8(qc, qs, wI, kc, ks, pos0, 4, 1024)
    ref = B.indexer_topk(qI, wI, KI, pos0, 4, 1024)   # the bf16 selection, for the overlap figure only
    torch.cuda.synchronize()
    idx, ref = idx.cpu().numpy(), ref.cpu().numpy()
    overlap, und = [], []
    for b in range(8):
        okc, oks = O.quantize_rows_fp8(np64(KI[b]).astype(np.float32))
        oqc, oqs = O.quantize_rows_fp8(np64(qI[b, 0]).astype(np.float32))
        I = O.indexer_scores_fp8(oqc[None], oqs[None], np64(wI[b]), okc, oks, pos0, 4)[0]
        bound = fp8_refined_bound(oqc, oqs, np64(wI[b, 0]), okc, oks, N, 1024, I)
        und.append(check_topk_row_bounded(idx[b, 0], I, bound, N, 1024, what=f"b{b}"))
        overlap.append(len(set(idx[b, 0].tolist()) & set(ref[b, 0].tolist())) / 1024)
    msg = (f"fp8 decode 1M: undecided entries per row {und}; fp8 vs bf16 selection overlap "
           f"{[round(o, 3) for o in overlap]}")
    say("  " + msg)
    warnings.warn(ParityCount(msg))


# ----------------------------------------------------------------------------- FP4 (E2M1) indexer

@pytest.mark.parametrize("dtype,rows,dim", [("bf16", 1000, 128), ("f32", 333, 64), ("bf16", 9, 1024)])
def test_quantize_fp4(dtype, rows, dim):
    say("quantize_fp4", dtype, rows, dim)
    x = gen(73, "q4.x", (rows, dim), dtype, std=2.0)
    x[1] = 0.0
    codes, scales = B.quantize_fp4(x)
    torch.cuda.synchronize()
    oc, osc = O.quantize_rows_fp4(np64(x).astype(np.float32))
    assert np.array_equal(codes.cpu().numpy(), O.pack_nibbles(oc))
    assert np.array_equal(scales.cpu().numpy(), osc)


def _unpack(packed_row):
    p = np.asarray(packed_row, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (2 * p.shape[-1],), dtype=np.uint8)
    out[..., 0::2], out[..., 1::2] = p & 0xF, p >> 4
    return out


@pytest.mark.parametrize("bt,Tq,N,HI,dI,pos0,m,k", [
    (2, 300, 2000, 64, 128, 4 * 2000 - 300, 4, 256),   # prefill route, ragged tail
    (1, 77, 5000, 20, 64, 16000, 4, 100),             # dI 64, HI not a multiple of 32
    (3, 5, 70000, 64, 128, 4 * 70000, 4, 1024),       # decode route, two-kernel top-k
    (1, 2, 3000, 128, 128, 3000 * 4 - 2, 4, 2048),    # 128 heads, max k
    (1, 1024, 7000, 64, 128, 4 * 7000 - 1024, 4, 512),  # spans of 3 and 4 key tiles, partial last tiles
])
def test_indexer_fp4(bt, Tq, N, HI, dI, pos0, m, k):
    """FP4 scores and top-k against the oracle on its own quantisation. E2M1 dot products are exact,
    so the selection is held to the same 1e-6 tie band as the bf16 path."""
    say("indexer fp4", bt, Tq, N, HI, dI, pos0, m, k)
    qI = gen(33, "i4.q", (bt, Tq, HI, dI))
    KI = gen(33, "i4.k", (bt, N, dI))
    wI = uniform_device(33, "i4.w", (bt, Tq, HI), DEV)
    qc, qs = B.quantize_fp4(qI)
    kc, ks = B.quantize_fp4(KI)
    sc = B.indexer_scores_fp4(qc, qs, wI, kc, ks, pos0, m)
    idx = B.indexer_topk_fp4(qc, qs, wI, kc, ks, pos0, m, k)
    torch.cuda.synchronize()
    sc, idx = sc.cpu().numpy(), idx.cpu().numpy()
    rows = range(Tq) if Tq <= 80 else sorted(set(np.linspace(0, Tq - 1, 40).astype(int)) | {0, Tq - 1})
    n_band = 0
    for b in range(bt):
        okc, oks = O.quantize_rows_fp4(np64(KI[b]).astype(np.float32))
        assert np.array_equal(okc, _unpack(kc[b].cpu().numpy()))
        for r in rows:
            oqc, oqs = O.quantize_rows_fp4(np64(qI[b, r]).astype(np.float32))
            I = O.indexer_scores_fp4(oqc[None], oqs[None], np64(wI[b, r:r + 1]), okc, oks, pos0 + r, m)[0]
            V = O.visible(pos0 + r, m, N)
            if V == 0:
                continue
            assert np.abs(sc[b, r, :V] - I[:V]).max() <= 1e-5 * np.abs(I[:V]).max(), (b, r)
            n_band += check_topk_row(idx[b, r], I, V, k, what=f"b{b} r{r}")
    say("  tie-band differences:", n_band)


@pytest.mark.parametrize("fmt", ["mxfp4", "mxfp8"])
@pytest.mark.parametrize("dtype,rows,dim", [("bf16", 300, 128), ("f32", 77, 1024), ("bf16", 5, 32)])
def test_quantize_mx(fmt, dtype, rows, dim):
    """MX-FP4 codes and E8M0 block scales bit-exact against the oracle, with zero, tiny, huge and
    saturating blocks among normal ones."""
    say("quantize", fmt, dtype, rows, dim)
    x = gen(35, "mx.x", (rows, dim), dtype).float()
    x = x * torch.exp2(torch.arange(rows, device=DEV, dtype=torch.float32) % 41 - 20)[:, None]
    x[0, :32] = 0.0                       # all-zero block
    if rows > 2:
        x[1, :32] = 2.0 ** -130           # exponent below -127: clamped scale, codes round to 0
        x[2, :32] = 3.0e30                # large exponent
        x[2, 5] = -0.0
    x = x.to(torch.bfloat16 if dtype == "bf16" else torch.float32)
    codes, sc = (B.quantize_mxfp4 if fmt == "mxfp4" else B.quantize_mxfp8)(x)
    torch.cuda.synchronize()
    oc, osc = (O.quantize_rows_mxfp4 if fmt == "mxfp4" else O.quantize_rows_mxfp8)(np64(x).astype(np.float32))
    assert np.array_equal(sc.cpu().numpy(), osc)
    got = codes.cpu().numpy()
    assert np.array_equal(_unpack(got) if fmt == "mxfp4" else got, oc)


@pytest.mark.parametrize("bt,Tq,N,HI,pos0,m,k", [
    (2, 300, 2000, 64, 4 * 2000 - 300, 4, 256),        # prefill route, ragged tail
    (1, 1024, 7000, 64, 4 * 7000 - 1024, 4, 512),      # spans of 3 and 4 key tiles
    (1, 77, 5000, 20, 16000, 4, 100),                  # HI not a multiple of 32
    (3, 5, 70000, 64, 4 * 70000, 4, 1024),             # decode route, two-kernel top-k
    (1, 2, 3000, 128, 3000 * 4 - 2, 4, 2048),          # 128 heads, max k
])
@pytest.mark.parametrize("fmt", ["mxfp4", "mxfp8"])
def test_indexer_mx(fmt, bt, Tq, N, HI, pos0, m, k):
    """MX-FP4 / MX-FP8 scores within the derived bound of the oracle on its own quantisation
    (dI = 128); top-k exact outside the bound."""
    say("indexer", fmt, bt, Tq, N, HI, pos0, m, k)
    qz, score, topk = ((B.quantize_mxfp4, B.indexer_scores_mxfp4, B.indexer_topk_mxfp4) if fmt == "mxfp4" else
                       (B.quantize_mxfp8, B.indexer_scores_mxfp8, B.indexer_topk_mxfp8))
    oqz, oscore, obound = ((O.quantize_rows_mxfp4, O.indexer_scores_mxfp4, mxfp4_score_bound) if fmt == "mxfp4" else
                           (O.quantize_rows_mxfp8, O.indexer_scores_mxfp8, mxfp8_score_bound))
    unpack = _unpack if fmt == "mxfp4" else (lambda a: a)
    dI = 128
    qI = gen(37, "mx.q", (bt, Tq, HI, dI))
    KI = gen(37, "mx.k", (bt, N, dI))
    wI = uniform_device(37, "mx.w", (bt, Tq, HI), DEV)
    qc, qs = qz(qI)
    kc, ks = qz(KI)
    sc = score(qc, qs, wI, kc, ks, pos0, m)
    idx = topk(qc, qs, wI, kc, ks, pos0, m, k)
    torch.cuda.synchronize()
    sc, idx = sc.cpu().numpy(), idx.cpu().numpy()
    rows = range(Tq) if Tq <= 80 else sorted(set(np.linspace(0, Tq - 1, 40).astype(int)) | {0, Tq - 1})
    n_band, worst = 0, 0.0
    for b in range(bt):
        okc, oks = oqz(np64(KI[b]).astype(np.float32))
        assert np.array_equal(okc, unpack(kc[b].cpu().numpy())) and np.array_equal(oks, ks[b].cpu().numpy())
        for r in rows:
            oqc, oqs = oqz(np64(qI[b, r]).astype(np.float32))
            I = oscore(oqc[None], oqs[None], np64(wI[b, r:r + 1]), okc, oks, pos0 + r, m)[0]
            V = O.visible(pos0 + r, m, N)
            if V == 0:
                continue
            bound = (obound(oqc, oqs, np64(wI[b, r]), okc, oks, V) if fmt == "mxfp4" else
                     mxfp8_refined_bound(oqc, oqs, np64(wI[b, r]), okc, oks, V, k, I))
            err = np.abs(sc[b, r, :V] - I[:V])
            assert (err <= bound).all(), (b, r, float((err / bound).max()))
            worst = max(worst, float((err / bound).max()))
            n_band += check_topk_row_bounded(idx[b, r], I, bound, V, k, what=f"b{b} r{r}")
    msg = f"{fmt} {bt}x{Tq}x{N} k={k}: undecided entries {n_band}; largest error / bound {worst:.3g}"
    say("  " + msg)
    warnings.warn(ParityCount(msg))



def test_indexer_fp4_decode_1m():
    say("indexer fp4 decode 1M: batch 8, 262144 keys")
    N, pos0 = 262144, 1 << 20
    qI = gen(4, "i4d.q", (8, 1, 64, 128))
    KI = gen(4, "i4d.k", (8, N, 128))
    wI = uniform_device(4, "i4d.w", (8, 1, 64), DEV)
    qc, qs = B.quantize_fp4(qI)
    kc, ks = B.quantize_fp4(KI)
    idx = B.indexer_topk_fp4(qc, qs, wI, kc, ks, pos0, 4, 1024)
    ref = B.indexer_topk(qI, wI, KI, pos0, 4, 1024)   # the bf16 selection, for the overlap figure only
    torch.cuda.synchronize()
    idx, ref = idx.cpu().numpy(), ref.cpu().numpy()
    overlap = []
    for b in range(8):
        okc, oks = O.quantize_rows_fp4(np64(KI[b]).astype(np.float32))
        oqc, oqs = O.quantize_rows_fp4(np64(qI[b, 0]).astype(np.float32))
        I = O.indexer_scores_fp4(oqc[None], oqs[None], np64(wI[b]), okc, oks, pos0, 4)[0]
        check_topk_row(idx[b, 0], I, N, 1024, what=f"b{b}")
        overlap.append(len(set(idx[b, 0].tolist()) & set(ref[b, 0].tolist())) / 1024)
    say("  fp4 vs bf16 selection overlap per row:", [round(o, 3) for o in overlap])


@pytest.mark.parametrize("fmt", ["mxfp4", "mxfp8"])
def test_indexer_mx_decode_1m(fmt):
    """MX top-k at the decode shape (batch 8 x 262144 keys at position 2^20, k = 1024), exact outside
    the derived score bound; two calls give identical indices."""
    say("indexer", fmt, "decode 1M: batch 8, 262144 keys")
    N, pos0 = 262144, 1 << 20
    qI = gen(8, "mxd.q", (8, 1, 64, 128))
    KI = gen(8, "mxd.k", (8, N, 128))
    wI = uniform_device(8, "mxd.w", (8, 1, 64), DEV)
    qz, topk = (B.quantize_mxfp4, B.indexer_topk_mxfp4) if fmt == "mxfp4" else (B.quantize_mxfp8, B.indexer_topk_mxfp8)
    oqz, oscore, obound = ((O.quantize_rows_mxfp4, O.indexer_scores_mxfp4, mxfp4_score_bound) if fmt == "mxfp4" else
                           (O.quantize_rows_mxfp8, O.indexer_scores_mxfp8, mxfp8_score_bound))
    qc, qs = qz(qI)
    kc, ks = qz(KI)
    idx = topk(qc, qs, wI, kc, ks, pos0, 4, 1024)
    idx2 = topk(qc, qs, wI, kc, ks, pos0, 4, 1024)
    torch.cuda.synchronize()
    assert torch.equal(idx, idx2)
    idx = idx.cpu().numpy()
    n_band = 0
    for b in range(8):
        okc, oks = oqz(np64(KI[b]).astype(np.float32))
        oqc, oqs = oqz(np64(qI[b, 0]).astype(np.float32))
        I = oscore(oqc[None], oqs[None], np64(wI[b]), okc, oks, pos0, 4)[0]
        bound = (obound(oqc, oqs, np64(wI[b, 0]), okc, oks, N) if fmt == "mxfp4" else
                 mxfp8_refined_bound(oqc, oqs, np64(wI[b, 0]), okc, oks, N, 1024, I))
        n_band += check_topk_row_bounded(idx[b, 0], I, bound, N, 1024, what=f"b{b}")
    msg = f"{fmt} decode 1M: undecided entries over 8 rows {n_band}"
    say("  " + msg)
    warnings.warn(ParityCount(msg))


# ----------------------------------------------------------------------------- attention

def _random_idx(bt, Tq, pos0, m, N, k, seed):
    rng = np.random.default_rng(seed)
    idx = -np.ones((bt, Tq, k), dtype=np.int32)
    for b in range(bt):
        for j in range(Tq):
            V = O.visible(pos0 + j, m, N)
            if V <= k:
                idx[b, j, :V] = np.arange(V)
            else:
                idx[b, j] = np.sort(rng.choice(V, size=k, replace=False))
    return idx


@pytest.mark.parametrize("dtype,mode,bt,Tq,N,pos0,m,k,w,H,d,rope,roo,sink", [
    ("f32", "csa", 1, 96, 32, 0, 4, 16, 16, 4, 64, 16, True, True),
    ("bf16", "csa", 2, 70, 64, 0, 4, 24, 16, 16, 64, 16, True, True),
    ("bf16", "hca", 2, 50, 40, 128 * 10, 128, 0, 128, 20, 128, 32, False, True),
    ("bf16", "csa", 1, 33, 3000, 4 * 2900, 4, 1024, 128, 64, 512, 64, True, True),
    ("bf16", "hca", 1, 40, 200, 128 * 180, 128, 0, 128, 32, 512, 64, True, False),
    ("bf16", "csa", 1, 20, 500, 1990, 4, 100, 7, 8, 256, 0, False, True),
    ("f32", "hca", 2, 30, 10, 0, 4, 0, 5, 3, 96, 32, True, True),
    ("bf16", "hca", 2, 41, 300, 128 * 250, 128, 0, 128, 64, 512, 64, True, True),
    ("bf16", "csa", 1, 37, 90, 0, 4, 256, 16, 64, 512, 64, True, False),
    ("bf16", "csa", 2, 9, 400, 4 * 390, 4, 64, 128, 64, 512, 64, False, True),
    ("bf16", "csa", 1, 20, 200, 4 * 150, 4, 16, 8, 64, 512, 64, True, True),   # one key tile (16 + 8 keys)
    ("bf16", "csa", 2, 10, 300, 4 * 290, 4, 64, 16, 64, 512, 64, False, True),  # three key tiles (64 + 16 keys)
    ("bf16", "hca", 2, 33, 150, 128 * 120, 128, 0, 64, 32, 512, 64, True, True),  # odd Tq: a half-empty 2-query block
    ("bf16", "csa", 1, 12, 300, 4 * 250, 4, 128, 32, 40, 512, 64, True, True),  # 40 heads: a partly empty head group
    # HCA with 49-64 heads of 512 dims: window-only rows from position 0, a partly empty head group without
    # sinks, and a two-tile key list with RoPE on 16 dims and no output de-rotation
    ("bf16", "hca", 1, 70, 5, 0, 128, 0, 16, 56, 512, 64, True, True),
    ("bf16", "hca", 2, 20, 40, 128 * 30, 128, 0, 24, 50, 512, 16, False, False),
    # 32 heads: four queries per workgroup, the last block with 2 of 4 queries
    ("bf16", "hca", 1, 6, 80, 128 * 60, 128, 0, 128, 32, 512, 64, True, True),
    ("bf16", "hca", 2, 13, 50, 128 * 20, 128, 0, 32, 24, 512, 32, True, False),
    ("bf16", "hca", 2, 3, 70, 128 * 60, 128, 0, 128, 32, 512, 64, True, True),  # 3 queries: two per workgroup
])
def test_attention_prefill(dtype, mode, bt, Tq, N, pos0, m, k, w, H, d, rope, roo, sink):
    say("attention", dtype, mode, bt, Tq, N, pos0, m, k, w, H, d, rope, roo, sink)
    q = gen(31, "at.q", (bt, Tq, H, d), dtype)
    kv = gen(31, "at.kv", (bt, N, d), dtype)
    wp0 = max(0, pos0 - w + 1)
    win = gen(31, "at.win", (bt, pos0 + Tq - wp0, d), dtype)
    sk = normal_device(31, "at.sink", (H,), 1.0, "f32", DEV) if sink else None
    idx = torch.from_numpy(_random_idx(bt, Tq, pos0, m, N, k, 3)).to(DEV) if mode == "csa" else None
    o, lse = B.compressed_attn_prefill(B.CSA if mode == "csa" else B.HCA, q, kv, idx, win, wp0, sk, pos0, m, w,
                                       k=k, rope_dims=rope, rope_on_output=roo, return_lse=True)
    torch.cuda.synchronize()
    for b in range(bt):
        ro, rl = O.attention(np64(q[b]), np64(kv[b]), np64(win[b]), wp0, pos0, m, w,
                             idx=idx[b].cpu().numpy() if idx is not None else None,
                             sink=np64(sk) if sink else None, rope_dims=rope, rope_on_output=roo)
        err = np.abs(np64(o[b]) - ro).max()
        lerr = np.abs(np64(lse[b]) - rl).max()
        say(f"  b{b}: max|o err| {err:.3g}  max|lse err| {lerr:.3g}")
        assert err <= ATOL[dtype] and lerr <= ATOL[dtype] * 5


@pytest.mark.parametrize("mode,Tq", [("hca", 6), ("csa", 1)])
def test_attention_logits_outgrow_reference(mode, Tq):
    """Logits that rise far above the first tiles': the first 64 entries are 100x smaller,
    and a sharp softmax scale makes later logits exceed the early maximum by far more than
    2^64 (base 2), so the kernel's softmax reference must move (and O be rescaled) many
    times. Queries are used as given (no RMSNorm, no RoPE), so the bf16 operands are exact
    and logits of this size carry only fp32 summation error."""
    say("attention outgrow", mode, Tq)
    bt, H, d, m, w, N = 1, 64, 512, (4 if mode == "csa" else 128), 16, 400
    pos0 = N * m
    k = 256 if mode == "csa" else 0
    q = gen(43, "og.q", (bt, Tq, H, d))
    kv = gen(43, "og.kv", (bt, N, d))
    kv[:, :64] *= 0.01
    win = gen(43, "og.win", (bt, pos0 + Tq - (pos0 - w + 1), d)) * 0.01
    sk = normal_device(43, "og.sink", (H,), 1.0, "f32", DEV)
    idx = torch.from_numpy(_random_idx(bt, Tq, pos0, m, N, k, 5)).to(DEV) if mode == "csa" else None
    if idx is not None:
        idx[..., :64] = torch.arange(64, device=DEV, dtype=idx.dtype)  # the first tile holds small entries
        idx = torch.sort(idx, dim=-1).values
    scale = 40.0 / np.sqrt(d)
    md = B.CSA if mode == "csa" else B.HCA
    kw = dict(k=k, rope_dims=0, apply_q_norm=False, scale=scale, return_lse=True)
    o, lse = B.compressed_attn_prefill(md, q, kv, idx, win, pos0 - w + 1, sk, pos0, m, w, **kw)
    od, lsed = B.compressed_attn_decode(md, q, kv, idx, win, pos0 - w + 1, sk, pos0, m, w, n_splits=3, **kw)
    torch.cuda.synchronize()
    ro, rl = O.attention(np64(q[0]), np64(kv[0]), np64(win[0]), pos0 - w + 1, pos0, m, w,
                         idx=idx[0].cpu().numpy() if idx is not None else None, sink=np64(sk), scale=scale,
                         apply_q_norm=False, rope_dims=0)
    assert rl.max() - 0.0 > 64 / np.log2(np.e)  # the logits really do outgrow any early reference
    for out, l in ((o, lse), (od, lsed)):
        err = np.abs(np64(out[0]) - ro).max()
        say(f"  max|o err| {err:.3g}")
        assert err <= 2e-2
        assert np.abs(np64(l[0]) - rl).max() <= 1e-1


# ----------------------------------------------------------------------------- FP8 KV storage

@pytest.mark.parametrize("dtype,bt,n,d,rope", [("bf16", 2, 37, 512, 64), ("f32", 1, 20, 128, 32),
                                               ("bf16", 1, 9, 256, 0)])
def test_quantize_kv_fp8(dtype, bt, n, d, rope):
    say("quantize_kv_fp8", dtype, bt, n, d, rope)
    x = gen(75, "kv8.x", (bt, n, d), dtype) * torch.logspace(-3, 3, n, device=DEV)[None, :, None].to(TD[dtype])
    x[0, 1] = 0.0
    rows, sc = B.quantize_kv_fp8(x, rope)
    torch.cuda.synchronize()
    rows, sc = rows.cpu(), sc.cpu().numpy()
    for b in range(bt):
        codes, rp, osc = O.quantize_kv_fp8(np64(x[b]), rope)
        assert np.array_equal(rows[b, :, : d - rope].numpy(), codes)
        gpu_rope = rows[b, :, d - rope:].contiguous().view(torch.bfloat16).float().numpy().astype(np.float64)
        assert np.array_equal(gpu_rope, rp)
        assert np.array_equal(sc[b].astype(np.float64), osc)


def _kv8_oracle(kv_raw_b, rope):
    codes, rp, osc = O.quantize_kv_fp8(np64(kv_raw_b), rope)
    return O.dequantize_kv_fp8(codes, rp, osc)


@pytest.mark.parametrize("mode,bt,Tq,N,pos0,m,k,w,H,d,rope", [
    ("csa", 1, 33, 3000, 4 * 2900, 4, 1024, 128, 64, 512, 64),
    ("hca", 2, 40, 200, 128 * 180, 128, 0, 128, 32, 512, 64),
    ("csa", 2, 50, 64, 0, 4, 24, 16, 16, 64, 16),
    ("hca", 1, 20, 50, 128 * 40, 128, 0, 16, 16, 128, 32),
    ("csa", 1, 17, 40, 4 * 30, 4, 16, 8, 16, 64, 0),
    ("csa", 1, 9, 500, 4 * 400, 4, 256, 32, 64, 512, 0),
    ("hca", 1, 12, 100, 128 * 90, 128, 0, 32, 32, 512, 32),
    ("csa", 2, 5, 300, 4 * 250, 4, 64, 40, 64, 512, 16),
])
def test_attention_kv8_prefill_and_decode(mode, bt, Tq, N, pos0, m, k, w, H, d, rope):
    """Attention over an FP8 + BF16 KV cache equals the oracle's attention over its own
    dequantisation of the same entries (prefill, and decode of the last query row)."""
    say("attention kv8", mode, bt, Tq, N, pos0, m, k, w, H, d, rope)
    q = gen(37, "a8.q", (bt, Tq, H, d))
    kv = gen(37, "a8.kv", (bt, N, d))
    wp0 = max(0, pos0 - w + 1)
    win = gen(37, "a8.win", (bt, pos0 + Tq - wp0, d))
    sk = normal_device(37, "a8.sink", (H,), 1.0, "f32", DEV)
    idx = torch.from_numpy(_random_idx(bt, Tq, pos0, m, N, k, 4)).to(DEV) if mode == "csa" else None
    md = B.CSA if mode == "csa" else B.HCA
    rows, sc = B.quantize_kv_fp8(kv, rope)
    ws = None
    if mode == "hca":  # entries widened once into a workspace; the tile route must agree bit for bit
        ws = torch.empty(B.lib().cskv_prefill_kv8_workspace_size(md, bt, N, d), dtype=torch.uint8, device=DEV)
        ot = B.compressed_attn_prefill(md, q, rows, idx, win, wp0, sk, pos0, m, w, k=k, rope_dims=rope,
                                       kv_scale=sc, workspace=torch.empty(0, dtype=torch.uint8, device=DEV))
    o = B.compressed_attn_prefill(md, q, rows, idx, win, wp0, sk, pos0, m, w, k=k, rope_dims=rope, kv_scale=sc,
                                  workspace=ws)
    if ws is not None:
        torch.cuda.synchronize()
        assert torch.equal(o.view(torch.int16), ot.view(torch.int16)), "workspace and tile routes differ"
        wide = ws.view(torch.bfloat16).view(bt, N, d)
        for b in range(bt):  # the widened entries are the exact dequantisation
            assert np.array_equal(np64(wide[b]), _kv8_oracle(kv[b], rope))
    last = Tq - 1
    od = B.compressed_attn_decode(md, q[:, last:].contiguous(), rows, idx[:, last:].contiguous() if idx is not None
                                  else None, win, wp0, sk, pos0 + last, m, w, k=k, rope_dims=rope, kv_scale=sc)
    torch.cuda.synchronize()
    for b in range(bt):
        deq = _kv8_oracle(kv[b], rope)
        ro, _ = O.attention(np64(q[b]), deq, np64(win[b]), wp0, pos0, m, w,
                            idx=idx[b].cpu().numpy() if idx is not None else None, sink=np64(sk), rope_dims=rope)
        err = np.abs(np64(o[b]) - ro).max()
        derr = np.abs(np64(od[b, 0]) - ro[last]).max()
        say(f"  b{b}: max|o err| {err:.3g}, decode row {derr:.3g}")
        assert err <= ATOL["bf16"] and derr <= ATOL["bf16"]


@pytest.mark.parametrize("mode,H", [("csa", 64), ("hca", 64), ("csa", 40), ("hca", 24)])
def test_decode_splits_and_prefill_agree(mode, H):
    """Every split count (staged fp32 partials, merged) and the single pass agree with the oracle;
    40 and 24 heads leave part of the last 16-head group empty."""
    say("decode splits", mode, H)
    bt, d, m, w = 3, 512, (4 if mode == "csa" else 128), 128
    N = 6000
    pos0 = N * m
    k = 1024 if mode == "csa" else 0
    q = gen(41, "dc.q", (bt, 1, H, d))
    kv = gen(41, "dc.kv", (bt, N, d))
    win = gen(41, "dc.win", (bt, w, d))
    sk = normal_device(41, "dc.sink", (H,), 1.0, "f32", DEV)
    idx = torch.from_numpy(_random_idx(bt, 1, pos0, m, N, k, 9)).to(DEV) if mode == "csa" else None
    md = B.CSA if mode == "csa" else B.HCA
    kw = dict(k=k, rope_dims=64, return_lse=True)
    outs = [B.compressed_attn_prefill(md, q, kv, idx, win, pos0 - w + 1, sk, pos0, m, w, **kw)]
    for ns in (1, 3, 7, 0, 64):
        outs.append(B.compressed_attn_decode(md, q, kv, idx, win, pos0 - w + 1, sk, pos0, m, w, n_splits=ns, **kw))
    torch.cuda.synchronize()
    for b in range(bt):
        ro, rl = O.attention(np64(q[b]), np64(kv[b]), np64(win[b]), pos0 - w + 1, pos0, m, w,
                             idx=idx[b].cpu().numpy() if idx is not None else None, sink=np64(sk), rope_dims=64)
        for i, (o, l) in enumerate(outs):
            err = np.abs(np64(o[b]) - ro).max()
            assert err <= 2e-2, (b, i, err)
            assert np.abs(np64(l[b]) - rl).max() <= 1e-1
    for o, l in outs[1:]:  # every split count agrees with the single pass to fp32-merge rounding
        assert (o.float() - outs[0][0].float()).abs().max().item() <= 1.6e-2


# ----------------------------------------------------------------------------- whole layers

def _attend_row(L, t, b, r, sel):
    """The GPU attention of query row r of sequence b over the selection `sel` (an oracle top-k row),
    on the caches and window rows the layer call left on the GPU."""
    kv = t.get("post.cache.kv", t["cache.kv"])[b:b + 1]
    win = t.get("post.win", t["win"])[b:b + 1]
    q = t["q"][b:b + 1, r:r + 1].contiguous()
    idx = torch.from_numpy(np.asarray(sel, dtype=np.int32)).to(DEV).reshape(1, 1, -1)
    kw = dict(k=L.k, rope_dims=L.rope_dims, rope_on_output=True, return_lse=True)
    if L.decode:
        o, l = B.compressed_attn_decode(B.CSA, q, kv, idx, win, L.win_pos0, t["sink"], L.pos0 + r, L.m, L.w,
                                        n_splits=L.n_splits, **kw)
    else:
        o, l = B.compressed_attn_prefill(B.CSA, q, kv, idx, win, L.win_pos0, t["sink"], L.pos0 + r, L.m, L.w, **kw)
    torch.cuda.synchronize()
    return np64(o[0, 0]), np64(l[0, 0])


def _check_layer(L, t, rows_per_seq, atol, max_band_rows=0.25):
    """Every sampled row is compared. Where the GPU's top-k differs from the oracle's inside the tie
    band (both are valid selections), the GPU attention is run again for that row on the oracle's
    selection and compared with the oracle's output, so no row goes unchecked and no GPU output
    feeds the oracle."""
    out, lse = t["out"], t["lse"]
    gidx = t["idx"].cpu().numpy() if L.kind == "csa" else None
    compared = alt = 0
    for b in range(L.batch):
        rows = rows_per_seq(L)
        o, l, idx, ex = oracle_layer(L, t, b, rows)
        for n, r in enumerate(rows):
            go, gl = np64(out[b, r]), np64(lse[b, r])
            if L.kind == "csa":
                I = ex["scores"][r]
                V = O.visible(L.pos0 + r, L.m, L.N)
                band = 1e-6 * abs(np.sort(I[:V])[::-1][min(L.k, V) - 1]) if V > 0 else 0.0
                band += key_rounding_band(np64(t["qI"][b, r]), np64(t["wI"][b, r]), ex.get("ik_new_exact"), L.dtype)
                check_topk_row(gidx[b, r], I, V, L.k, band=band, what=f"b{b} r{r}")
                if not np.array_equal(gidx[b, r], idx[r]):
                    go, gl = _attend_row(L, t, b, r, idx[r])
                    alt += 1
            err = np.abs(go - o[n]).max()
            assert err <= atol, f"{L.name} b{b} row {r}: max err {err:.3g}"
            assert np.abs(gl - l[n]).max() <= 5 * atol
            compared += 1
    msg = (f"{L.name}: {compared} rows compared, {alt} of them (GPU top-k != oracle's inside the tie band) "
           f"on the oracle's selection")
    say("  " + msg)
    warnings.warn(ParityCount(msg))
    assert alt <= max_band_rows * compared


def _run(L):
    """Run the layer; return its inputs with the caches and window as they were before the call
    (and, under "post.", as the call left them)."""
    t = LY.make_inputs(L)
    pre = {k: t[k].clone() for k in ("cache.kv", "cache.ik", "win") if k in t}
    LY.run_layer(L, t)
    torch.cuda.synchronize()
    res = dict(t)
    res.update({f"post.{k}": t[k] for k in pre})
    res.update(pre)
    return res


def test_tiny_csa_f32_end_to_end():
    L = LY.tiny_csa("f32")
    say("tiny CSA f32 end to end", L)
    t = _run(L)
    _check_layer(L, t, lambda L: list(range(L.T)), 1e-4, max_band_rows=0.02)


def test_tiny_csa_bf16_end_to_end():
    L = LY.tiny_csa("bf16")
    say("tiny CSA bf16 end to end")
    t = _run(L)
    _check_layer(L, t, lambda L: list(range(L.T)), 2e-2, max_band_rows=0.05)


@pytest.mark.parametrize("kind", ["csa", "hca"])
def test_chunked_layer_small(kind):
    m = 4 if kind == "csa" else 128
    L = LY.LayerCall(kind, 2, 700, 128 * 40, 128 * 40 // m, d=512, H=20, m=m, w=128, k=256, HI=64, dI=128,
                     seed=8, name=f"small.{kind}")
    say("chunked small", L)
    t = _run(L)
    _check_layer(L, t, lambda L: sorted({0, 1, 2, 3, 127, 128, 129, 255, 256, 400, 511, 512, 698, 699}), 2e-2)


@pytest.mark.parametrize("kind", ["csa", "hca"])
def test_streaming_decode_grows_caches_like_prefill(kind):
    """Decode a sequence token by token from empty caches: the caches the stream appends
    must equal a one-shot prefill's, and every step must match the oracle's row."""
    say("streaming decode", kind)
    m, T = (4, 96) if kind == "csa" else (8, 96)
    L = LY.LayerCall(kind, 2, T, 0, 0, d=64, rope_dims=16, H=4, m=m, w=16, k=16, HI=4, dI=32, seed=77,
                     name=f"stream.{kind}")
    t = LY.make_inputs(L)
    LY.run_layer(L, t)  # reference: the whole sequence at once
    S = LY.DecodeStream(dataclasses.replace(L, T=1), capacity=T // m)
    biases = {nm: v for nm, v in t.items() if nm.endswith(".B")}
    outs, lses, idxs = [], [], []
    row = lambda nm, p: t[nm][:, p:p + 1].contiguous()
    for p in range(T):
        for nm in S.ring:
            S.slot(nm, p).copy_(t[nm][:, p])  # the producer's rows of token p
        o = S.step(p, row("q", p), row("win_raw", p), t["sink"], biases,
                   qI=row("qI", p) if kind == "csa" else None, wI=row("wI", p) if kind == "csa" else None)
        outs.append(o.clone())
        lses.append(S.lse.clone())
        if kind == "csa":
            idxs.append(S.idx.clone())
    torch.cuda.synchronize()
    assert S.n_entries == T // m
    for tag in S.cache:
        assert torch.equal(S.cache[tag], t[f"cache.{tag}"]), tag
    td = dict(t)
    td["out"], td["lse"] = torch.cat(outs, 1), torch.cat(lses, 1)
    if kind == "csa":
        td["idx"] = torch.cat(idxs, 1)
    _check_layer(L, td, lambda L: list(range(T)), ATOL["bf16"])


def test_window_ring_equals_linear_window():
    """A window kept as a ring of w rows (row p mod w, win_pos0 = 0) gives the same result as
    the same rows laid out in position order."""
    say("window ring")
    bt, H, d, w, N, m, k = 2, 8, 128, 16, 300, 4, 32
    pos0 = 4 * N - 5                      # window positions pos0 - 15 .. pos0, wrapping the ring
    q = gen(81, "wr.q", (bt, 1, H, d))
    kv = gen(81, "wr.kv", (bt, N, d))
    lin = gen(81, "wr.win", (bt, w, d))   # positions pos0 - w + 1 .. pos0 in order
    ring = torch.empty_like(lin)
    for i in range(w):
        ring[:, (pos0 - w + 1 + i) % w] = lin[:, i]
    sink = normal_device(81, "wr.sink", (H,), 1.0, "f32", DEV)
    idx = torch.tensor(_random_idx(bt, 1, pos0, m, N, k, 5), dtype=torch.int32, device=DEV)
    for mode in (B.CSA, B.HCA):
        a = B.compressed_attn_decode(mode, q, kv, idx, lin, pos0 - w + 1, sink, pos0, m, w, k=k, rope_dims=64)
        r = B.compressed_attn_decode(mode, q, kv, idx, ring, 0, sink, pos0, m, w, k=k, rope_dims=64)
        torch.cuda.synchronize()
        assert torch.equal(a, r), mode


def test_prefill_from_scratch_edges():
    # rows before the first complete block see the window only; T not a multiple of m
    L = LY.LayerCall("csa", 1, 301, 0, 0, d=128, rope_dims=32, H=16, m=4, w=9, k=8, HI=32, dI=64, seed=9,
                     name="edge")
    say("edge prefill", L)
    t = _run(L)
    _check_layer(L, t, lambda L: list(range(L.T)), 2e-2, max_band_rows=0.05)


def test_layer_is_deterministic():
    L = LY.LayerCall("csa", 1, 2048, 0, 0, d=512, H=64, m=4, w=128, k=256, HI=64, dI=128, seed=10, name="det")
    t = LY.make_inputs(L)
    a = LY.run_layer(L, t).clone()
    ia = t["idx"].clone()
    b = LY.run_layer(L, t)
    torch.cuda.synchronize()
    assert torch.equal(a, b) and torch.equal(ia, t["idx"])


# ----------------------------------------------------------------------------- full-size workloads

def test_hca_prefill_16k_sampled():
    L = LY.hca_prefill_16k()
    say("HCA prefill 16k", L)
    t = _run(L)
    _check_layer(L, t, lambda L: sorted({0, 126, 127, 128, 255, 256, 8191, 8192, 16383} |
                                         set(np.random.default_rng(0).choice(L.T, 24, replace=False).tolist())), 2e-2)


def test_csa_prefill_64k_sampled():
    L = LY.csa_prefill_64k()
    say("CSA prefill 64k", L)
    t = _run(L)
    _check_layer(L, t, lambda L: sorted({0, 3, 4095, 4096, 4099, 32768, 65535} |
                                         set(np.random.default_rng(1).choice(L.T, 16, replace=False).tolist())), 2e-2)


def test_decode_1m_full():
    for L in LY.decode_1m():
        say("decode 1M", L)
        t = _run(L)
        _check_layer(L, t, lambda L: [0], 2e-2, max_band_rows=0.25)


def test_chunked_prefill_512k_sampled():
    for L in LY.chunked_prefill_512k():
        say("chunked prefill 512k", L.name, L.kind)
        t = _run(L)
        _check_layer(L, t, lambda L: sorted({0, 1, 127, 128, 2048, 4095} |
                                             set(np.random.default_rng(2).choice(L.T, 4, replace=False).tolist())), 2e-2)


def test_indexer_topk_matches_its_two_halves():
    # indexer_topk chunks its rows through a bounded workspace; the result must equal
    # indexer_scores + topk_select over the whole matrix, bit for bit
    say("indexer_topk == indexer_scores + topk_select")
    bt, Tq, N, HI, dI, k = 2, 3000, 20000, 64, 128, 512
    pos0 = N * 4 - Tq
    qI = gen(51, "h2.q", (bt, Tq, HI, dI))
    KI = gen(51, "h2.k", (bt, N, dI))
    wI = uniform_device(51, "h2.w", (bt, Tq, HI), DEV)
    a = B.indexer_topk(qI, wI, KI, pos0, 4, k)
    sc = B.indexer_scores(qI, wI, KI, pos0, 4)
    b = B.topk_select(sc, N, pos0, 4, k)
    torch.cuda.synchronize()
    assert B.indexer_workspace_bytes(bt, Tq, N, HI, k, B.BF16) < bt * Tq * B.score_ld(N) * 4  # it did chunk
    assert torch.equal(a, b)



@pytest.mark.parametrize("dtype,bt,Tq,N,HI,dI,pos0,m", [
    ("bf16", 1, 77, 5000, 20, 64, 16000, 4),   # several key spans per row, partial last tiles
    ("bf16", 2, 300, 400, 64, 128, 0, 4),      # one span, rows with no visible entry
    ("bf16", 3, 5, 70000, 64, 128, 4 * 70000, 4),  # decode-shaped rows
    ("f32", 1, 100, 128, 2, 32, 0, 4),
    ("fp8", 1, 1024, 7000, 64, 128, 4 * 7000 - 1024, 4),  # spans of 3 and 4 key tiles
    ("fp8", 2, 300, 400, 20, 64, 0, 4),
    ("fp4", 1, 1024, 7000, 64, 128, 4 * 7000 - 1024, 4),
    ("fp4", 1, 77, 5000, 20, 64, 16000, 4),    # 32-byte key rows
    ("fp4", 3, 5, 70000, 64, 128, 4 * 70000, 4),
    ("mxfp4", 1, 1024, 7000, 64, 128, 4 * 7000 - 1024, 4),
    ("mxfp4", 3, 5, 70000, 20, 128, 4 * 70000, 4),
    ("mxfp8", 1, 1024, 7000, 64, 128, 4 * 7000 - 1024, 4),
    ("mxfp8", 3, 5, 70000, 20, 128, 4 * 70000, 4),
])
def test_indexer_scores_write_extent(dtype, bt, Tq, N, HI, dI, pos0, m):
    # every visible entry gets a finite score; past V_t only -inf may be written, and nothing
    # at or past the last row's V (the end of every swept key range) or past N is touched
    say("indexer_scores write extent", dtype, bt, Tq, N, HI, dI, pos0, m)
    lowp = dtype in ("fp8", "fp4", "mxfp4", "mxfp8")
    qI = gen(23, "we.q", (bt, Tq, HI, dI), "bf16" if lowp else dtype)
    KI = gen(23, "we.k", (bt, N, dI), "bf16" if lowp else dtype)
    wI = uniform_device(23, "we.w", (bt, Tq, HI), DEV)
    ld = B.score_ld(N) + 8
    sc = torch.full((bt, Tq, ld), float("nan"), dtype=torch.float32, device=DEV)
    if lowp:
        qz, fn = {"fp8": (B.quantize_fp8, B.indexer_scores_fp8), "fp4": (B.quantize_fp4, B.indexer_scores_fp4),
                  "mxfp4": (B.quantize_mxfp4, B.indexer_scores_mxfp4),
                  "mxfp8": (B.quantize_mxfp8, B.indexer_scores_mxfp8)}[dtype]
        (qc, qs), (kc, ks) = qz(qI), qz(KI)
        fn(qc, qs, wI, kc, ks, pos0, m, scores=sc)
    else:
        B.indexer_scores(qI, wI, KI, pos0, m, scores=sc)
    torch.cuda.synchronize()
    sc = sc.cpu()
    V = torch.tensor([O.visible(pos0 + r, m, N) for r in range(Tq)])
    vend = int(V.max())
    col = torch.arange(ld)
    for b in range(bt):
        x = sc[b]
        vis = col[None, :] < V[:, None]
        assert torch.isfinite(x[vis]).all(), f"b{b}: visible entry not written or not finite"
        mid = (~vis) & (col[None, :] < vend)
        assert (torch.isnan(x[mid]) | torch.isneginf(x[mid])).all(), f"b{b}: past V_t something other than -inf"
        assert torch.isnan(x[:, vend:]).all(), f"b{b}: written at or past the end of the swept range"


# ----------------------------------------------------------------------------- projections

def _gemm_bound(A, B, ref):
    """Per-element bound for a bf16 product with fp32 accumulation and a bf16 result: one bf16
    ulp of the exact value (the fp32 sum may sit across a rounding boundary) plus the fp32
    summation error over K terms."""
    K = A.shape[-1]
    mag = np.abs(A) @ np.abs(B)
    return 2.0 ** -8 * np.abs(ref) + K * 2.0 ** -24 * mag + 1e-30


@pytest.mark.parametrize("T,r,n_out", [(300, 256, 8192), (37, 64, 136), (129, 1536, 1024)])
def test_lowrank_proj(T, r, n_out):
    say("lowrank_proj", T, r, n_out)
    cq = gen(51, "lp.cq", (T, r))
    W = gen(51, "lp.W", (r, n_out), std=r ** -0.5)
    out = B.lowrank_proj(cq, W)
    torch.cuda.synchronize()
    a, w = np64(cq), np64(W)
    ref = O.lowrank_proj(a, w)
    err = np.abs(np64(out) - ref)
    bound = _gemm_bound(a, w, ref)
    say(f"  max err {err.max():.3g}, max err/bound {(err / bound).max():.3g}")
    assert (err <= bound).all()


@pytest.mark.parametrize("T,H,d,G,dg,D", [(70, 64, 128, 8, 256, 512), (200, 64, 512, 8, 1024, 4096),
                                         (33, 16, 64, 4, 80, 136)])
def test_grouped_out_proj(T, H, d, G, dg, D):
    say("grouped_out_proj", T, H, d, G, dg, D)
    o = gen(52, "gp.o", (T, H, d))
    Wg = gen(52, "gp.Wg", (G, (H // G) * d, dg), std=((H // G) * d) ** -0.5)
    Wo = gen(52, "gp.Wo", (G * dg, D), std=(G * dg) ** -0.5)
    y, mid = B.grouped_out_proj(o, Wg, Wo, return_mid=True)
    torch.cuda.synchronize()
    o64, wg, wo = np64(o), np64(Wg), np64(Wo)
    # stage 1 against the oracle, per group
    ref_mid = O.grouped_out_proj_mid(o64, wg)
    og = o64.reshape(T, G, (H // G) * d)
    for g in range(G):
        err = np.abs(np64(mid[:, g]) - ref_mid[:, g])
        assert (err <= _gemm_bound(og[:, g], wg[g], ref_mid[:, g])).all(), g
    # stage 2 on the GPU's own intermediate (identical inputs), against the oracle's final product
    m64 = np64(mid)
    ref_y = m64.reshape(T, G * dg) @ wo
    err = np.abs(np64(y) - ref_y)
    bound = _gemm_bound(m64.reshape(T, G * dg), wo, ref_y)
    say(f"  y: max err {err.max():.3g}, max err/bound {(err / bound).max():.3g}")
    assert (err <= bound).all()
    # and the whole chain against the oracle end to end (bf16 intermediate on both sides)
    full = O.grouped_out_proj(o64, wg, wo)
    assert np.abs(np64(y) - full).max() <= 2e-2 * max(1.0, np.abs(full).max())
