"""Host-side helpers for the GPU parity tests: comparisons and the oracle
pipeline of one layer call. Everything here runs on the CPU; the oracle
only ever sees the seeded inputs (copied from where the generator drew them),
never an output of the GPU path."""
from __future__ import annotations

import math
from typing import Dict, Iterable, Optional

import numpy as np

from oracle import cskv_oracle as O


class ParityCount(UserWarning):
    """How many rows an end-to-end parity check compared, and how (shown in pytest's summary)."""


def np64(t) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def bf16_ulp(x: np.ndarray) -> np.ndarray:
    """Spacing of bf16 values at |x| (2**-133 below the normal range)."""
    _, e = np.frexp(np.abs(x))
    return np.ldexp(1.0, np.maximum(e - 8, -133))


def assert_storage_close(gpu: np.ndarray, exact: np.ndarray, dtype: str, what: str, rtol_f32=1e-5):
    """bf16: within one bf16 ulp of the exact (fp64) value, plus 2**-17 of the RMS of its row.

    f32: within 1e-5 of (|x| + RMS of its row). A compressed entry is a
    weighted sum of up to m' rows; its fp32 rounding error scales with the
    magnitude of the summed terms, i.e. the row's scale, not with the
    (possibly cancelled) element itself. In bf16 the final rounding adds at
    most half an ulp of the result; the fp32 error before it (a few dozen
    fp32 ulps of the row's scale, 2**-17 ~ 64 * 2**-23) matters only where a
    channel's weighted sum cancels to far below the terms (about one element
    in 4e5 on N(0,1) streams).
    """
    err = np.abs(gpu - exact)
    if dtype == "bf16":
        rms = np.sqrt(np.mean(exact * exact, axis=-1, keepdims=True))
        bad = err > bf16_ulp(exact) * (1 + 1e-9) + 2.0 ** -17 * rms
        assert not bad.any(), (f"{what}: {bad.sum()} of {bad.size} elements beyond 1 bf16 ulp + 2^-17 row rms, "
                               f"max err {err.max():.3g}")
    else:
        rms = np.sqrt(np.mean(exact * exact, axis=-1, keepdims=True))
        bad = err > rtol_f32 * (np.abs(exact) + rms)
        assert not bad.any(), f"{what}: {bad.sum()} elements beyond 1e-5 (|x| + row rms), max err {err.max():.3g}"


def check_topk_row(gpu_row: np.ndarray, scores: np.ndarray, V: int, k: int, band: float = None,
                   what: str = "") -> int:
    """Checks one row of selected indices against oracle scores.

    Bit-exact outside the tie band: every entry scoring above I_k + band must
    be selected and none scoring below I_k - band; the row is ascending,
    distinct, visible, and -1 padded. Returns how many selected entries fall
    inside the band but differ from the oracle's own pick.
    """
    gpu_row = np.asarray(gpu_row, dtype=np.int64)
    if V <= k:
        exp = np.concatenate([np.arange(V), -np.ones(k - V, dtype=np.int64)])
        assert np.array_equal(gpu_row, exp), f"{what}: V={V} <= k={k} must list all visible entries"
        return 0
    assert (gpu_row >= 0).all() and (gpu_row < V).all(), f"{what}: out-of-range index"
    assert (np.diff(gpu_row) > 0).all(), f"{what}: not strictly ascending"
    ref = O.topk_row(scores, V, k)
    s = scores[:V]
    Ik = np.sort(s)[::-1][k - 1]
    if band is None:
        band = 1e-6 * abs(Ik)
    sel = np.zeros(V, dtype=bool)
    sel[gpu_row] = True
    must_in = s > Ik + band
    must_out = s < Ik - band
    assert sel[must_in].all(), f"{what}: {int((~sel[must_in]).sum())} entries above the band missing"
    assert not sel[must_out].any(), f"{what}: {int(sel[must_out].sum())} entries below the band selected"
    return len(set(gpu_row.tolist()) ^ set(ref.tolist())) // 2


def fp8_score_bound(q_codes, q_scales, w_row, k_codes, k_scales, V: int) -> np.ndarray:
    """Bound on |I_gpu - I| for one query's FP8 scores over keys 0..V-1.

    Measured on gfx950 (in-bounds probes of v_mfma_f32_32x32x64_f8f6f4 and
    v_mfma_f32_32x32x16_fp8_fp8): the products held in 8 consecutive bytes of
    one lane's operand -- here 8 consecutive dims -- are summed on a grid of
    2**(E - 13), E the exponent of the group's largest product; finer bits are
    dropped. So each of the 7 other products of a group loses less than
    2**-13 * (group max), and the group max is at most the product of the two
    rows' maxima over the group. fp32 sums of the 16 group sums and of the
    heads add at most 2**-20 * sum |products| and 2**-17 * |terms|. ReLU is
    1-Lipschitz, so per key s:
      B[s] = ks[s] * sum_h |w_h qs_h| * (7 * 2**-13 * sum_g Qmax[h,g] Kmax[s,g]
                                        + 2**-20 * (|dq_h| . |dk_s|) + 2**-17 * |dq_h . dk_s|)
    """
    return e4m3_group_bound(O.e4m3_decode(q_codes), O.e4m3_decode(k_codes[:V]),
                            np.asarray(w_row, dtype=np.float64) * np.asarray(q_scales, dtype=np.float64),
                            np.asarray(k_scales[:V], dtype=np.float64))


def mxfp8_score_bound(q_codes, q_scales, w_row, k_codes, k_scales, V: int) -> np.ndarray:
    """Bound on |I_gpu - I| for one query's MX-FP8 scores over keys 0..V-1: the FP8 group model
    (fp8_score_bound) on the decoded rows, whose 8-value groups lie inside one 32-value block and so
    share one scale (the grid moves with it); the block-sum additions (at most an fp32 ulp each,
    measured for the block-scaled instruction) fall under its 2**-20 * sum |products| term."""
    dq = O.dequantize_mxfp8(q_codes, q_scales)
    dk = O.dequantize_mxfp8(k_codes[:V], k_scales[:V])
    return e4m3_group_bound(dq, dk, np.asarray(w_row, dtype=np.float64), np.ones(V))


def fp8_refined_bound(q_codes, q_scales, w_row, k_codes, k_scales, V: int, k: int, scores,
                      cap: int = 8192) -> np.ndarray:
    """fp8_score_bound, taken product by product (e4m3_product_bound) for the entries near the k-th
    score whose top-k membership depends on it."""
    b = fp8_score_bound(q_codes, q_scales, w_row, k_codes, k_scales, V)
    dq = O.e4m3_decode(q_codes)
    wq = np.asarray(w_row, dtype=np.float64) * np.asarray(q_scales, dtype=np.float64)
    kc, ks = np.asarray(k_codes), np.asarray(k_scales, dtype=np.float64)
    return refine_bound_near_kth(scores, b, V, k, lambda ix: e4m3_product_bound(dq, O.e4m3_decode(kc[ix]), wq, ks[ix]),
                                 cap)


def mxfp8_refined_bound(q_codes, q_scales, w_row, k_codes, k_scales, V: int, k: int, scores,
                        cap: int = 8192) -> np.ndarray:
    """mxfp8_score_bound, taken product by product for the entries near the k-th score."""
    b = mxfp8_score_bound(q_codes, q_scales, w_row, k_codes, k_scales, V)
    dq = O.dequantize_mxfp8(q_codes, q_scales)
    kc, ks = np.asarray(k_codes), np.asarray(k_scales)
    return refine_bound_near_kth(scores, b, V, k, lambda ix: e4m3_product_bound(
        dq, O.dequantize_mxfp8(kc[ix], ks[ix]), w_row, np.ones(ix.size)), cap)


def e4m3_group_bound(dq, dk, wq, ks) -> np.ndarray:
    """The FP8 error model of fp8_score_bound on decoded rows dq [HI, dI], dk [V, dI], head factors
    wq [HI] (weight times row scale) and key factors ks [V]."""
    V = dk.shape[0]
    HI, dI = dq.shape
    qmax = np.abs(dq).reshape(HI, dI // 8, 8).max(axis=2)
    kmax = np.abs(dk).reshape(V, dI // 8, 8).max(axis=2)
    gm = kmax @ qmax.T                          # [V, HI]
    ab = np.abs(dk) @ np.abs(dq).T
    dot = np.abs(dk @ dq.T)
    per = 7 * 2.0 ** -13 * gm + 2.0 ** -20 * ab + 2.0 ** -17 * dot
    return np.asarray(ks, dtype=np.float64) * (per @ np.abs(np.asarray(wq, dtype=np.float64)))


def e4m3_product_bound(dq, dk, wq, ks, chunk: int = 512) -> np.ndarray:
    """The group model of fp8_score_bound taken product by product, for the keys in dk.

    Each E4M3 x E4M3 product is exact in float64. In a group of 8 products the
    grid is 2**(E - 13), E = floor(log2) of the group's largest |product|; a
    product on that grid loses nothing, and one off it loses less than the
    grid step: its remainder r below the grid when bits are cut toward zero,
    g - r when cut toward minus infinity, at most g / 2 when rounded, so
    max(r, g - r) covers all three. The fp32 sums of the group sums and of the
    heads add the same 2**-20 * sum |products| + 2**-17 * |dot| as before.
    dq [HI, dI], dk [n, dI] decoded rows, wq [HI] head factors, ks [n] key
    factors; returns [n].
    """
    dq = np.asarray(dq, dtype=np.float64)
    dk = np.asarray(dk, dtype=np.float64)
    HI, dI = dq.shape
    aw = np.abs(np.asarray(wq, dtype=np.float64))
    out = np.empty(dk.shape[0])
    for a in range(0, dk.shape[0], chunk):
        kk = dk[a:a + chunk]
        n = kk.shape[0]
        P = np.abs(kk[:, None, :] * dq[None, :, :]).reshape(n, HI, dI // 8, 8)
        gm = P.max(axis=-1, keepdims=True)
        _, ex = np.frexp(gm)                                   # gm = f * 2**ex, f in [0.5, 1)
        g = np.ldexp(1.0, ex - 14)                             # 2**(E - 13), E = ex - 1
        r = np.fmod(P, g)
        per = np.where(r > 0, np.maximum(r, g - r), 0.0).sum(axis=(-1, -2))   # [n, HI]
        ab = np.abs(kk) @ np.abs(dq).T
        dot = np.abs(kk @ dq.T)
        out[a:a + n] = (per + 2.0 ** -20 * ab + 2.0 ** -17 * dot) @ aw
    return np.asarray(ks, dtype=np.float64) * out


def refine_bound_near_kth(scores, bound, V: int, k: int, product_bound, cap: int = 16384) -> np.ndarray:
    """Tighten a per-entry bound where the top-k decision depends on it.

    Entries whose interval [s - b, s + b] meets the span of the still-undecided
    entries (see check_topk_row_bounded) get product_bound(indices) instead,
    when smaller; at most `cap` of them, nearest the k-th score. Both bounds
    hold for every entry, so the result does too.
    """
    b = np.array(bound[:V], dtype=np.float64)
    if V <= k:
        return b
    s = np.asarray(scores[:V], dtype=np.float64)
    und = undecided_mask(s, b, k)
    if not und.any():
        return b
    lo, hi = (s - b)[und].min(), (s + b)[und].max()
    near = np.nonzero((s + b >= lo) & (s - b <= hi))[0]
    if near.size > cap:
        Ik = np.sort(s)[::-1][k - 1]
        near = near[np.argsort(np.abs(s[near] - Ik))[:cap]]
    b[near] = np.minimum(b[near], product_bound(near))
    return b


def undecided_mask(s, b, k: int) -> np.ndarray:
    """Entries that the bounds leave undecided: some k others may beat them, yet not k surely do."""
    V = s.shape[0]
    lo, hi = s - b, s + b
    n_reach = V - np.searchsorted(np.sort(hi), lo, side="left") - 1
    n_above = V - np.searchsorted(np.sort(lo), hi, side="right")
    return ~((n_reach < k) | (n_above >= k))


def check_topk_row_bounded(gpu_row: np.ndarray, scores: np.ndarray, bound: np.ndarray, V: int, k: int,
                           what: str = "") -> int:
    """Checks a selection made from scores known only within +-bound per entry.

    An entry must be selected when fewer than k others can reach its lowest
    possible score, and must not be when at least k others surely exceed its
    highest; entries in between may go either way. The row must be ascending,
    distinct, visible and -1 padded. Returns the number of undecided entries.
    """
    gpu_row = np.asarray(gpu_row, dtype=np.int64)
    if V <= k:
        exp = np.concatenate([np.arange(V), -np.ones(k - V, dtype=np.int64)])
        assert np.array_equal(gpu_row, exp), f"{what}: V={V} <= k={k} must list all visible entries"
        return 0
    assert (gpu_row >= 0).all() and (gpu_row < V).all(), f"{what}: out-of-range index"
    assert (np.diff(gpu_row) > 0).all(), f"{what}: not strictly ascending"
    s = np.asarray(scores[:V], dtype=np.float64)
    lo, hi = s - bound[:V], s + bound[:V]
    hi_sorted = np.sort(hi)
    lo_sorted = np.sort(lo)
    n_reach = V - np.searchsorted(hi_sorted, lo, side="left") - 1   # others with hi >= my lo
    n_above = V - np.searchsorted(lo_sorted, hi, side="right")      # entries with lo > my hi
    must_in = n_reach < k
    must_out = n_above >= k
    sel = np.zeros(V, dtype=bool)
    sel[gpu_row] = True
    assert sel[must_in].all(), f"{what}: {int((~sel[must_in]).sum())} certain entries missing"
    assert not sel[must_out].any(), f"{what}: {int(sel[must_out].sum())} excluded entries selected"
    return int(V - must_in.sum() - must_out.sum())


def oracle_layer(L, t, b: int, rows: Iterable[int]):
    """Oracle pipeline of one layer call for sequence b at the given query rows.

    t holds the seeded device inputs of the call (make_inputs) with the caches
    and window buffer as they were BEFORE the call; slices are copied to the
    host as float64. Returns (o [len(rows), H, d], lse [len(rows), H],
    idx [Tq, k] filled at the rows, extras). Compressed entries and window
    rows are rounded to the storage type, as the cache stores them.
    """
    rnd = O.round_bf16 if L.dtype == "bf16" else (lambda x: x)
    h = lambda name: np64(t[name][b])
    opt = lambda name: np64(t[name][b]) if name in t else None
    rows = list(rows)
    def cache(name, n_valid):
        # rows past n_valid are written by the call itself (and recomputed below); never read them
        full = t[name][b]
        a = np.zeros(tuple(full.shape), dtype=np.float64)
        a[:n_valid] = np64(full[:n_valid])
        return a

    kv = cache("cache.kv", L.n_cached)
    ik = cache("cache.ik", L.n_cached) if L.kind == "csa" else None
    extras = {}
    if L.n_new:
        if L.kind == "csa":
            new = O.csa_compress(h("kv.Ca"), h("kv.Cb"), h("kv.Za"), h("kv.Zb"), np64(t["kv.B"]), L.m, L.pos0,
                                 opt("kv.prevCb"), opt("kv.prevZb"), apply_norm=True, rope_dims=L.rope_dims)
            kv[L.n_cached:] = rnd(new)
            newk = O.csa_compress(h("ik.Ca"), h("ik.Cb"), h("ik.Za"), h("ik.Zb"), np64(t["ik.B"]), L.m, L.pos0,
                                  opt("ik.prevCb"), opt("ik.prevZb"))
            extras["ik_new_exact"] = newk
            ik[L.n_cached:] = rnd(newk)
        else:
            new = O.hca_compress(h("kv.C"), h("kv.Z"), np64(t["kv.B"]), L.m, L.pos0, apply_norm=True,
                                 rope_dims=L.rope_dims)
            kv[L.n_cached:] = rnd(new)
    win = cache("win", L.win_cached)
    win[L.win_cached:] = rnd(O.prepare_window(h("win_raw"), L.pos0, rope_dims=L.rope_dims))
    sink = np64(t["sink"])
    idx = np.full((L.T, L.k), -1, dtype=np.int64) if L.kind == "csa" else None
    extras["scores"] = {}
    outs, lses = [], []
    for r in rows:
        rid = None
        if L.kind == "csa":
            qI = np64(t["qI"][b, r:r + 1])
            wI = np64(t["wI"][b, r:r + 1])
            I = O.indexer_scores(qI, wI, ik, L.pos0 + r, L.m)[0]
            extras["scores"][r] = I
            idx[r] = O.topk_row(I, O.visible(L.pos0 + r, L.m, L.N), L.k)
            rid = idx[r:r + 1]
        # one query row at absolute position pos0 + r (a one-row call of the same definition)
        o, l = O.attention(np64(t["q"][b, r:r + 1]), kv, win, L.win_pos0, L.pos0 + r, L.m, L.w, idx=rid,
                           sink=sink, rope_dims=L.rope_dims)
        outs.append(o[0])
        lses.append(l[0])
    return np.stack(outs), np.stack(lses), idx, extras


def key_rounding_band(qI_row: np.ndarray, wI_row: np.ndarray, ik_new_exact: Optional[np.ndarray],
                      dtype: str = "bf16") -> float:
    """Largest change of one indexer score when every recomputed key element moves by one storage ulp.

    |dI_s| <= sum_h |w_h| * sum_c |q_hc| * ulp(K_sc) (ReLU is 1-Lipschitz). Stored
    cache entries are identical on both sides and add nothing. In fp32 the
    compressor's own rounding (a few fp32 ulps) stands in for the storage ulp.
    """
    if ik_new_exact is None or ik_new_exact.size == 0:
        return 0.0
    if dtype == "bf16":
        u = bf16_ulp(np.abs(ik_new_exact)).max(axis=0)  # per channel, worst entry
    else:
        u = np.abs(ik_new_exact).max(axis=0) * 2.0 ** -21
    return float(np.sum(np.abs(wI_row)[:, None] * np.abs(qI_row) * u[None, :]))


def mxfp4_score_bound(q_codes, q_scales, w_row, k_codes, k_scales, V: int) -> np.ndarray:
    """Bound on |I_gpu - I| for one query's MX-FP4 scores over keys 0..V-1.

    Each 32-value block's sum of E2M1 products is a multiple of 1/4 below
    32 * 36 and exact in fp32; an in-bounds probe of
    v_mfma_scale_f32_32x32x64_f8f6f4 showed the instruction adding the two
    scaled block sums of one k-step with up to one fp32 ulp of truncation,
    and the second k-step adds to that in fp32. So each head's dot product is
    off by at most 3 * 2**-23 * A[h, s], A = sum over blocks of |scaled block
    sum|; ReLU is 1-Lipschitz and the fp32 head sum adds at most
    HI * 2**-24 * sum_h |w_h dot_h|:
      B[s] = sum_h |w_h| (3 * 2**-23 A[h, s] + HI * 2**-24 |dot_h[s]|)
    """
    dq = O.dequantize_mxfp4(q_codes, q_scales)          # [HI, dI]
    dk = O.dequantize_mxfp4(k_codes[:V], k_scales[:V])  # [V, dI]
    HI, dI = dq.shape
    nb = dI // O.MX_BLOCK
    blk = np.einsum("hbk,sbk->shb", dq.reshape(HI, nb, -1), dk.reshape(V, nb, -1))  # [V, HI, blocks]
    A = np.abs(blk).sum(axis=2)
    dot = np.abs(blk.sum(axis=2))
    w = np.abs(np.asarray(w_row, dtype=np.float64))
    return (3 * 2.0 ** -23 * A + HI * 2.0 ** -24 * dot) @ w
