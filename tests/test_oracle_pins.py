"""Pins for the CPU oracle: closed forms, invariants, brute force and library cross-checks.

The pages print no worked numeric example, so every pin below is a value the
definitions fix exactly (hand-derived closed forms), a property that must
hold for any input, a brute-force recount on tiny inputs, or a cross-check
against an independent library routine. Each is chosen so that a plausible
slip in the oracle (swapped bias halves, a b-block off by one, a sink with a
value vector, a wrong RoPE pairing, a transposed operand) fails at least one.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import cskv_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
rng = np.random.default_rng(1234)


# ---------------------------------------------------------------- compression

def test_csa_hand_closed_form():
    # m = 2, one channel. Entry 0 pools only its own a-block (no block before it);
    # entry 1 pools a-rows 2,3 and b-rows 0,1 under one softmax.
    Ca = np.array([[1.0], [2.0], [3.0], [4.0]])
    Cb = np.array([[10.0], [20.0], [30.0], [40.0]])
    Z = np.zeros((4, 1))
    B = np.zeros((4, 1))
    out = O.csa_compress(Ca, Cb, Z, Z, B, m=2)
    assert np.allclose(out[:, 0], [1.5, (3 + 4 + 10 + 20) / 4], rtol=0, atol=1e-15)
    # A bias of ln 2 on the first b-row (row 0 of the stacked [B^b; B^a]) doubles its weight.
    B[0, 0] = math.log(2.0)
    out = O.csa_compress(Ca, Cb, Z, Z, B, m=2)
    assert np.allclose(out[:, 0], [1.5, (2 * 10 + 20 + 3 + 4) / 5], rtol=0, atol=1e-14)
    # The same bias on the first a-row (row m) acts on entry 0 as well.
    B[:] = 0
    B[2, 0] = math.log(3.0)
    out = O.csa_compress(Ca, Cb, Z, Z, B, m=2)
    assert np.allclose(out[:, 0], [(3 * 1 + 2) / 4, (3 * 3 + 4 + 10 + 20) / 6], rtol=0, atol=1e-14)


def test_csa_weights_sum_to_one_shift_and_onehot():
    m, c, T = 4, 5, 32
    Za, Zb = rng.normal(size=(T, c)) * 3, rng.normal(size=(T, c)) * 3
    B = rng.normal(size=(2 * m, c))
    for i in range(T // m):
        S = O.csa_weights(Za, Zb, B, m, i)
        assert S.shape[0] == (m if i == 0 else 2 * m)
        assert np.allclose(S.sum(axis=0), 1.0, atol=1e-12)
    # Constant input -> constant output (weights sum to one), for any logits.
    ones = np.ones((T, c)) * 2.5
    out = O.csa_compress(ones, ones, Za, Zb, B, m)
    assert np.allclose(out, 2.5, atol=1e-12)
    # Shift invariance: adding the same constant to all 2m logits of a block changes nothing.
    Ca, Cb = rng.normal(size=(T, c)), rng.normal(size=(T, c))
    base = O.csa_compress(Ca, Cb, Za, Zb, B, m)
    assert np.allclose(O.csa_compress(Ca, Cb, Za + 7.0, Zb + 7.0, B, m), base, atol=1e-12)
    # One-hot: a huge logit on b-row 1 of block 2 (feeding entry 3) selects that row.
    Zb2 = Zb.copy()
    Zb2[2 * m + 1, :] = 1e4
    out = O.csa_compress(Ca, Cb, Za, Zb2, B, m)
    assert np.allclose(out[3], Cb[2 * m + 1], atol=1e-12)
    assert np.allclose(out[:3], base[:3]) and np.allclose(out[4:], base[4:])


def test_csa_m1_identity_and_uniform_pair():
    T, c = 9, 3
    Ca, Cb = rng.normal(size=(T, c)), rng.normal(size=(T, c))
    Za = rng.normal(size=(T, c))
    B = np.zeros((2, c))
    # b-stream masked out -> identity on C^a.
    out = O.csa_compress(Ca, Cb, Za, np.full((T, c), -np.inf), B, m=1)
    assert np.allclose(out, Ca, atol=1e-15)
    # Uniform weights: (C^a_i + C^b_{i-1}) / 2, and C^a_0 for the first entry.
    Z = np.zeros((T, c))
    out = O.csa_compress(Ca, Cb, Z, Z, B, m=1)
    assert np.allclose(out[0], Ca[0])
    assert np.allclose(out[1:], (Ca[1:] + Cb[:-1]) / 2, atol=1e-15)


def test_csa_chunk_with_tail_equals_full():
    m, c, T = 4, 6, 40
    Ca, Cb, Za, Zb = (rng.normal(size=(T, c)) for _ in range(4))
    B = rng.normal(size=(2 * m, c))
    full = O.csa_compress(Ca, Cb, Za, Zb, B, m, apply_norm=True, rope_dims=4)
    cut = 16
    part = O.csa_compress(Ca[cut:], Cb[cut:], Za[cut:], Zb[cut:], B, m, pos0=cut,
                          prev_Cb=Cb[cut - m:cut], prev_Zb=Zb[cut - m:cut], apply_norm=True, rope_dims=4)
    assert np.allclose(part, full[cut // m:], atol=1e-13)


def test_entry_rope_position_is_first_token_of_its_block():
    # One rotated pair (rope_dims = c = 2, so theta_0 = 1) and a raw entry of [1, 0]: the stored
    # entry is [cos p, sin p], p the entry's rotary position, which must be the first token of its
    # own block, pos0 + m * i. CSA: a-row 0 of each block takes all the weight and holds [1, 0].
    m, n, pos0 = 4, 5, 4 * 37
    Ca = np.tile([[1.0, 0.0], [0.0, 3.0], [0.0, 3.0], [0.0, 3.0]], (n, 1))
    Za = np.tile([[50.0, 50.0], [0.0, 0.0], [0.0, 0.0], [0.0, 0.0]], (n, 1))
    Zb = np.full((n * m, 2), -50.0)
    out = O.csa_compress(Ca, np.zeros_like(Ca), Za, Zb, np.zeros((2 * m, 2)), m, pos0=pos0,
                         prev_Cb=np.zeros((m, 2)), prev_Zb=np.full((m, 2), -50.0), rope_dims=2)
    p = pos0 + m * np.arange(n)
    assert np.allclose(out, np.stack([np.cos(p), np.sin(p)], axis=1), atol=1e-12)
    # HCA with uniform weights over a block of identical rows [1, 0]: entry i at pos0 + m' i
    mh, pos0h = 8, 8 * 11
    out = O.hca_compress(np.tile([1.0, 0.0], (3 * mh, 1)), None, None, mh, pos0=pos0h, rope_dims=2)
    p = pos0h + mh * np.arange(3)
    assert np.allclose(out, np.stack([np.cos(p), np.sin(p)], axis=1), atol=1e-12)
    # window rows (m' = 1), normed ([2, 0] has RMS sqrt 2) and each turned at its own position
    out = O.prepare_window(np.tile([2.0, 0.0], (4, 1)), 1000, eps=0.0, rope_dims=2)
    p = 1000 + np.arange(4)
    assert np.allclose(out, math.sqrt(2.0) * np.stack([np.cos(p), np.sin(p)], axis=1), atol=1e-12)


def test_hca_hand_closed_form_and_m1_identity():
    C = np.array([[1.0, -2.0], [3.0, 4.0]])
    Z = np.array([[0.0, 0.0], [math.log(3.0), 0.0]])
    out = O.hca_compress(C, Z, None, m=2)
    assert np.allclose(out[0], [(1 + 9) / 4, 1.0], atol=1e-15)
    # m' = 1: the softmax runs over a single row, so any weights give the identity.
    X = rng.normal(size=(7, 5))
    out = O.hca_compress(X, rng.normal(size=(7, 5)) * 10, rng.normal(size=(1, 5)), m=1)
    assert np.allclose(out, X, atol=1e-15)
    # Trailing partial block is not emitted.
    assert O.hca_compress(rng.normal(size=(300, 2)), None, None, m=128).shape == (2, 2)


def test_hca_uniform_is_block_mean():
    X = rng.normal(size=(256, 4))
    out = O.hca_compress(X, None, None, m=128)
    assert np.allclose(out, X.reshape(2, 128, 4).mean(axis=1), atol=1e-13)


def test_hca_positional_bias_enters_the_softmax():
    # The bias B[p] is added to the logit of row p of every block ("Paper Breakdown:
    # DeepSeek-V4", §2.3.2: softmax of Z + B over the block's m' rows).
    m, c = 4, 3
    X = rng.normal(size=(2 * m, c))
    # Z = -B cancels the bias: uniform weights, the block mean.
    Bv = rng.normal(size=(m, c)) * 3
    out = O.hca_compress(X, -np.tile(Bv, (2, 1)), Bv, m=m)
    assert np.allclose(out, X.reshape(2, m, c).mean(axis=1), atol=1e-13)
    # Z = 0 with one large bias per channel selects that row of each block, per channel.
    rows = np.array([0, 3, 1])
    Bh = np.zeros((m, c))
    Bh[rows, np.arange(c)] = 1e4
    out = O.hca_compress(X, None, Bh, m=m)
    expect = np.stack([X[i * m + rows, np.arange(c)] for i in range(2)])
    assert np.allclose(out, expect, atol=1e-12)
    # A bias of log(3) on row 1 only: weights 1:3:1:1 in every block.
    B3 = np.zeros((m, c))
    B3[1] = math.log(3.0)
    out = O.hca_compress(X, None, B3, m=m)
    w = np.array([1.0, 3.0, 1.0, 1.0]) / 6.0
    assert np.allclose(out, np.einsum("p,ipc->ic", w, X.reshape(2, m, c)), atol=1e-13)


# ---------------------------------------------------------- RMSNorm and RoPE

def test_rmsnorm_closed_form_and_unit_rms():
    assert np.allclose(O.rmsnorm(np.array([3.0, 4.0]), eps=0.0), [3 / math.sqrt(12.5), 4 / math.sqrt(12.5)])
    # eps joins the mean square under the root: mean 12.5 + 0.5 = 13
    assert np.allclose(O.rmsnorm(np.array([3.0, 4.0]), eps=0.5), [3 / math.sqrt(13.0), 4 / math.sqrt(13.0)],
                       rtol=0, atol=1e-15)
    X = rng.normal(size=(10, 64)) * 5
    Y = O.rmsnorm(X, eps=0.0)
    assert np.allclose(np.sqrt((Y * Y).mean(axis=-1)), 1.0, atol=1e-13)
    g = rng.uniform(size=64)
    assert np.allclose(O.rmsnorm(X, g, eps=0.0), Y * g)


def test_rope_matches_complex_rotation():
    d, dr, base = 12, 8, 10000.0
    x = rng.normal(size=(5, d))
    pos = np.array([0, 1, 7, 100, 65536])
    y = O.rope(x, pos, dr, base)
    assert np.array_equal(y[:, :d - dr], x[:, :d - dr])
    z = x[:, d - dr::2] + 1j * x[:, d - dr + 1::2]
    j = np.arange(dr // 2)
    z = z * np.exp(1j * pos[:, None] * base ** (-2.0 * j / dr))
    assert np.allclose(y[:, d - dr::2], z.real, atol=1e-12)
    assert np.allclose(y[:, d - dr + 1::2], z.imag, atol=1e-12)
    # Hand value: pair 0 turns by pos radians.
    v = O.rope(np.array([1.0, 0.0, 0.0, 1.0]), np.array(2), 4)
    assert np.allclose(v, [math.cos(2), math.sin(2), -math.sin(0.02), math.cos(0.02)])


def test_rope_norm_and_relative_position():
    d, dr = 16, 8
    q, k = rng.normal(size=d), rng.normal(size=d)
    for t, s, delta in [(10, 3, 5), (1000, 999, 77), (5, 40, 123456)]:
        a = O.rope(q, np.array(t), dr) @ O.rope(k, np.array(s), dr)
        b = O.rope(q, np.array(t + delta), dr) @ O.rope(k, np.array(s + delta), dr)
        assert abs(a - b) < 1e-10
        assert abs(np.linalg.norm(O.rope(q, np.array(t), dr)) - np.linalg.norm(q)) < 1e-12
    # Rotating by -t undoes rotating by t.
    assert np.allclose(O.rope(O.rope(q, np.array(33), dr), np.array(-33), dr), q, atol=1e-13)


# ------------------------------------------------------------ indexer, top-k

def test_indexer_hand_closed_form():
    qI = np.array([[[1.0, 0.0], [0.0, 1.0]]])
    wI = np.array([[2.0, 3.0]])
    KI = np.array([[1.0, 1.0], [-1.0, 2.0], [3.0, -1.0], [9.0, 9.0]])
    # query at t = 2 with m = 1 sees entries 0..2, not entry 3
    I = O.indexer_scores(qI, wI, KI, pos0=2, m=1)
    assert np.array_equal(I[0], [5.0, 6.0, 6.0, -np.inf])
    assert list(O.indexer_topk(qI, wI, KI, 2, 1, 2)[0]) == [1, 2]
    assert list(O.indexer_topk(qI, wI, KI, 2, 1, 1)[0]) == [1]
    assert list(O.indexer_topk(qI, wI, KI, 2, 1, 5)[0]) == [0, 1, 2, -1, -1]


def test_indexer_visibility_by_complete_blocks():
    KI = rng.normal(size=(10, 4))
    qI = rng.normal(size=(12, 2, 4))
    wI = rng.uniform(size=(12, 2))
    I = O.indexer_scores(qI, wI, KI, pos0=0, m=4)
    for t in range(12):
        V = (t + 1) // 4
        assert np.all(np.isfinite(I[t, :V])) and np.all(np.isneginf(I[t, V:]))


def test_indexer_brute_force_loops():
    Tq, HI, dI, N = 3, 3, 5, 7
    qI = rng.integers(-3, 4, size=(Tq, HI, dI)).astype(float)
    KI = rng.integers(-3, 4, size=(N, dI)).astype(float)
    wI = rng.uniform(size=(Tq, HI))
    I = O.indexer_scores(qI, wI, KI, pos0=100, m=4)
    for t in range(Tq):
        for s in range(N):
            ref = 0.0
            for h in range(HI):
                dot = sum(qI[t, h, c] * KI[s, c] for c in range(dI))
                ref += wI[t, h] * (dot if dot > 0 else 0.0)
            assert abs(I[t, s] - ref) < 1e-12


def test_topk_brute_force_with_ties():
    for trial in range(300):
        V = int(rng.integers(1, 14))
        k = int(rng.integers(1, 10))
        scores = rng.integers(0, 4, size=V).astype(float)  # many exact ties
        got = O.topk_row(np.concatenate([scores, [-np.inf] * 3]), V, k)
        if V <= k:
            ref = list(range(V)) + [-1] * (k - V)
        else:
            ranked = sorted(range(V), key=lambda s: (-scores[s], s))
            ref = sorted(ranked[:k])
        assert list(got) == ref
    # exhaustive check of the tie rule on one small case
    scores = np.array([0.5, 2, 2, 1, 2, 0])
    assert list(O.topk_row(scores, 6, 2)) == [1, 2]
    assert list(O.topk_row(scores, 6, 4)) == [1, 2, 3, 4]
    assert list(O.topk_row(scores, 2, 3)) == [0, 1, -1]


# ------------------------------------------------------------------ attention

def _mk_layer(T=24, d=16, dr=4, H=3, m=4, w=5, N=None, seed=0):
    r = np.random.default_rng(seed)
    N = T // m if N is None else N
    return dict(q=r.normal(size=(T, H, d)), kv=r.normal(size=(N, d)), win=r.normal(size=(T, d)),
                sink=r.normal(size=H), T=T, d=d, dr=dr, H=H, m=m, w=w)


def test_attention_hand_two_keys():
    # kv entries e0 = [1,0], e1 = [0,1]; query at t = 3, m = 2 -> both visible;
    # window w = 1 holds one zero row; scale 1, no norm/rope; sink 0.
    q = np.array([[[1.0, 0.0]]])
    kv = np.array([[1.0, 0.0], [0.0, 1.0]])
    win = np.zeros((4, 2))
    o, lse = O.attention(q, kv, win, 0, pos0=3, m=2, w=1, sink=np.array([0.0]), scale=1.0,
                         apply_q_norm=False, rope_dims=0, rope_on_output=False)
    e = math.e
    assert np.allclose(o[0, 0], [e / (e + 3), 1 / (e + 3)], atol=1e-15)
    assert abs(lse[0, 0] - math.log(e + 3)) < 1e-15


def test_attention_one_key_plus_sink_closed_form():
    # t = 0, m = 4: no compressed entry visible; the window holds only row 0.
    d = 8
    e0 = rng.normal(size=(1, d))
    q = rng.normal(size=(1, 2, d))
    z = np.array([0.3, -1.2])
    o, lse = O.attention(q, np.zeros((0, d)), e0, 0, pos0=0, m=4, w=4, sink=z, scale=0.5,
                         apply_q_norm=False, rope_dims=0, rope_on_output=False)
    l = (q[0] @ e0[0]) * 0.5
    sig = 1.0 / (1.0 + np.exp(z - l))
    assert np.allclose(o[0], sig[:, None] * e0[0][None, :], atol=1e-14)
    assert np.allclose(lse[0], np.logaddexp(z, l), atol=1e-14)


def test_attention_sink_scales_plain_softmax():
    L = _mk_layer()
    args = dict(pos0=0, m=L["m"], w=L["w"], rope_dims=L["dr"])
    o0, lse0 = O.attention(L["q"], L["kv"], L["win"], 0, sink=None, **args)
    o1, lse1 = O.attention(L["q"], L["kv"], L["win"], 0, sink=L["sink"], **args)
    frac = 1.0 / (1.0 + np.exp(L["sink"][None, :] - lse0))  # share of mass left to real keys
    assert np.allclose(o1, o0 * frac[..., None], atol=1e-13)
    assert np.allclose(lse1, np.logaddexp(lse0, L["sink"][None, :]), atol=1e-13)


def test_attention_no_sink_matches_torch_sdpa_fp64():
    L = _mk_layer(T=24, d=16, dr=0, H=3, m=4, w=5)
    T, H, d, m, w = L["T"], L["H"], L["d"], L["m"], L["w"]
    N = L["kv"].shape[0]
    o, _ = O.attention(L["q"], L["kv"], L["win"], 0, pos0=0, m=m, w=w, sink=None,
                       apply_q_norm=False, rope_dims=0, rope_on_output=False)
    keys = torch.from_numpy(np.concatenate([L["kv"], L["win"]]))  # [N + T, d]
    mask = torch.zeros(T, N + T, dtype=torch.bool)
    for t in range(T):
        mask[t, :(t + 1) // m] = True
        mask[t, N + max(0, t - w + 1):N + t + 1] = True
    qt = torch.from_numpy(L["q"]).permute(1, 0, 2)  # [H, T, d]
    ref = torch.nn.functional.scaled_dot_product_attention(
        qt, keys.expand(H, -1, -1), keys.expand(H, -1, -1), attn_mask=mask.expand(H, -1, -1))
    assert np.allclose(o, ref.permute(1, 0, 2).numpy(), atol=1e-12)


def test_csa_with_k_at_least_visible_equals_dense():
    L = _mk_layer(T=32, N=8)
    kw = dict(pos0=0, m=L["m"], w=L["w"], sink=L["sink"], rope_dims=L["dr"])
    idx = np.stack([O.topk_row(np.zeros(8), O.visible(t, L["m"], 8), 8) for t in range(32)])
    o_csa, l_csa = O.attention(L["q"], L["kv"], L["win"], 0, idx=idx, **kw)
    o_hca, l_hca = O.attention(L["q"], L["kv"], L["win"], 0, idx=None, **kw)
    assert np.allclose(o_csa, o_hca, atol=1e-14) and np.allclose(l_csa, l_hca, atol=1e-14)


def test_attention_rows_with_nothing_visible_are_window_only():
    L = _mk_layer(T=8, m=4)
    kw = dict(pos0=0, m=4, w=L["w"], sink=L["sink"], rope_dims=L["dr"])
    o_full, _ = O.attention(L["q"], L["kv"], L["win"], 0, **kw)
    o_win, _ = O.attention(L["q"], np.zeros((0, L["d"])), L["win"], 0, **kw)
    assert np.allclose(o_full[:3], o_win[:3])  # t = 0..2: V_t = 0
    assert not np.allclose(o_full[3], o_win[3])  # t = 3 sees entry 0


def test_attention_output_derotation_is_relative():
    # Shifting every position (query, entries, window) by the same amount leaves
    # logits and the de-rotated output unchanged: build the same layer twice.
    r = np.random.default_rng(5)
    d, dr, H, m, w = 16, 8, 2, 4, 4
    raw_kv, raw_win, q = r.normal(size=(3, d)), r.normal(size=(8, d)), r.normal(size=(1, H, d))
    outs = []
    for shift in (0, 4096):
        t = 11 + shift
        kv = O.rope(O.rmsnorm(raw_kv), np.array([0, 4, 8]) + shift, dr)
        win = O.rope(O.rmsnorm(raw_win), np.arange(t - 7, t + 1), dr)
        qt = O.prepare_query(q[0], t, True, None, 1e-6, dr, 10000.0)
        o, lse = O.attend_one(qt, np.concatenate([kv, win]), None, 0.25)
        outs.append((O.rope(o, np.full(H, -t), dr), lse))
    assert np.allclose(outs[0][0], outs[1][0], atol=1e-9)
    assert np.allclose(outs[0][1], outs[1][1], atol=1e-9)


def test_attention_self_key_closed_form_with_rope_and_window_offset():
    # One visible key: the window row of the query's own token (w = 1), in a window buffer that
    # starts at position win_pos0 = 5, with RoPE on every dim and the output de-rotated. The raw
    # row x has entries +-1, so with eps = 0 its RMSNorm is x itself. The stored row is
    # e = RoPE_t(x); the query (head 0: 5x, head 1: -x/2, normed to x and -x) becomes +-RoPE_t(x), so its logit is
    # +-scale * |x|^2 = +-scale * d whatever t is, and since the value is the key itself the output
    # is sigma(l - z) * e, which de-rotated by -t is sigma(l - z) * x. A query turned at another position, a window
    # read that ignores win_pos0, or an output turned forward instead of back all break it.
    r = np.random.default_rng(11)
    d, scale = 8, 0.3
    t, win_pos0 = 9, 5
    x = r.choice([-1.0, 1.0], size=d)
    raw = r.normal(size=(t - win_pos0 + 1, d))
    raw[-1] = x
    win = O.prepare_window(raw, win_pos0, eps=0.0, rope_dims=d)
    q = np.stack([5 * x, -x / 2])[None]                       # [1, 2, d]: RMSNorm gives x and -x
    z = np.array([0.4, -0.7])
    o, lse = O.attention(q, np.zeros((0, d)), win, win_pos0, pos0=t, m=4, w=1, sink=z, scale=scale,
                         eps=0.0, rope_dims=d, rope_on_output=True)
    ell = np.array([scale * d, -scale * d])
    sig = 1.0 / (1.0 + np.exp(z - ell))
    assert np.allclose(o[0], sig[:, None] * x[None, :], atol=1e-12)
    assert np.allclose(lse[0], np.logaddexp(z, ell), atol=1e-12)
    # without de-rotation the output is the stored (rotated) row itself
    o2, _ = O.attention(q, np.zeros((0, d)), win, win_pos0, pos0=t, m=4, w=1, sink=z, scale=scale,
                        eps=0.0, rope_dims=d, rope_on_output=False)
    assert np.allclose(o2[0], sig[:, None] * win[-1][None, :], atol=1e-12)
    assert not np.allclose(win[-1], x)


def test_attention_shift_invariance_through_oracle_caches():
    # Build one CSA layer twice from the same raw streams, once at positions 0.. and once shifted
    # by delta (a multiple of m): compressed entries and window rows come from the oracle's own
    # compressor and window preparation, the shifted cache holds delta/m extra entries in front
    # and the selected indices move with it. With the output de-rotated, every output and lse
    # must be unchanged: only relative positions may matter. Rows are compared from t = w - 1 on
    # (before that the unshifted window is cut at position 0); the shifted window buffer starts at
    # position delta + w - 1 - (w - 1) = delta, so a window read that ignores win_pos0 fails.
    r = np.random.default_rng(12)
    m, c, T, H, dr, w, k = 4, 16, 40, 3, 8, 6, 5
    delta = 4 * 1021
    Ca, Cb, Za, Zb = (r.normal(size=(T, c)) for _ in range(4))
    Bz = r.normal(size=(2 * m, c))
    raw_win = r.normal(size=(T, c))
    q = r.normal(size=(T, H, c))
    sink = r.normal(size=H)
    idx = np.full((T, k), -1)
    for j in range(T):
        V = O.visible(j, m, T // m)
        sel = np.sort(r.permutation(V)[:k])
        idx[j, :len(sel)] = sel
    res = []
    for shift in (0, delta):
        ent = O.csa_compress(Ca, Cb, Za, Zb, Bz, m, pos0=shift, apply_norm=True, rope_dims=dr)
        kv = np.concatenate([r.normal(size=(shift // m, c)), ent])
        win = O.prepare_window(raw_win, shift, rope_dims=dr)
        idx_s = np.where(idx >= 0, idx + shift // m, -1)
        rows = range(w - 1, T)
        res.append(O.attention(q, kv, win, shift, pos0=shift, m=m, w=w, idx=idx_s, sink=sink,
                               rope_dims=dr, rope_on_output=True, rows=rows))
    assert np.allclose(res[0][0], res[1][0], atol=1e-9)
    assert np.allclose(res[0][1], res[1][1], atol=1e-9)
    # and the pin is not vacuous: without de-rotation the two outputs differ
    raw = [O.attention(q, np.concatenate([r.normal(size=(s // m, c)),
                                          O.csa_compress(Ca, Cb, Za, Zb, Bz, m, pos0=s, apply_norm=True,
                                                         rope_dims=dr)]),
                       O.prepare_window(raw_win, s, rope_dims=dr), s, pos0=s, m=m, w=w,
                       idx=np.where(idx >= 0, idx + s // m, -1), sink=sink, rope_dims=dr,
                       rope_on_output=False, rows=[T - 1])[0] for s in (0, delta)]
    assert not np.allclose(raw[0], raw[1], atol=1e-3)


def test_decode_row_equals_prefill_row():
    L = _mk_layer(T=20)
    kw = dict(m=L["m"], w=L["w"], sink=L["sink"], rope_dims=L["dr"])
    o_all, l_all = O.attention(L["q"], L["kv"], L["win"], 0, pos0=0, **kw)
    for t in (0, 7, 19):
        o1, l1 = O.attention(L["q"][t:t + 1], L["kv"], L["win"], 0, pos0=t, **kw)
        assert np.allclose(o1[0], o_all[t]) and np.allclose(l1[0], l_all[t])


# -------------------------------------------------------------- storage type

def test_round_bf16_against_torch():
    x = np.concatenate([rng.normal(size=5000) * 10.0 ** rng.integers(-40, 38, size=5000),
                        [0.0, -0.0, 1.0, 3.0e38, -3.3e38, 1e-41]])
    ref = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).double().numpy()
    # torch rounds via float32; compare only where fp64 -> fp32 is exact enough not to double-round
    x32 = x.astype(np.float32).astype(np.float64)
    got = O.round_bf16(x32)
    assert np.array_equal(got, ref)


# ---------------------------------------------------------------- FP8 (E4M3) indexer

def _torch_e4m3(y):
    """torch's own float32 -> float8_e4m3fn conversion (an independent implementation)."""
    return torch.tensor(np.asarray(y, dtype=np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_e4m3_table_and_anchors():
    # every finite code decodes as torch's float8_e4m3fn does; spec anchors by hand
    t = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    d = O.e4m3_decode(np.arange(256))
    finite = ~np.isnan(t)
    assert np.array_equal(np.isnan(d), np.isnan(t))
    assert np.array_equal(d[finite], t[finite])
    for code, val in ((0x38, 1.0), (0x7E, 448.0), (0x08, 2.0 ** -6), (0x01, 2.0 ** -9), (0x40, 2.0),
                      (0x3C, 1.5), (0xB8, -1.0), (0x77, 240.0)):
        assert O.e4m3_decode(code) == val, hex(code)
        assert O.e4m3_encode(val) == code, hex(code)


def test_e4m3_encode_matches_torch_incl_ties():
    vals = O.e4m3_values()
    mids = (vals[:-1] + vals[1:]) / 2                          # exact ties: must go to the even code
    near = np.concatenate([np.nextafter(mids, 0), np.nextafter(mids, 1e9)])
    rnd = rng.uniform(-448, 448, 20000) * np.exp2(rng.integers(-14, 1, 20000))
    for y in (mids, -mids, near, -near, rnd, vals, -vals):
        y32 = np.asarray(y, dtype=np.float32)
        ok = np.abs(y32.astype(np.float64)) <= 448
        assert np.array_equal(O.e4m3_encode(y32[ok]), _torch_e4m3(y32[ok]))
    # ties land on even codes, and each midpoint is exactly between the two neighbours
    c = O.e4m3_encode(mids)
    assert (c % 2 == 0).all()
    assert O.e4m3_encode(500.0) == 0x7E and O.e4m3_encode(-1e6) == 0xFE   # saturation
    assert O.e4m3_encode(-0.0) == 0x80


def test_quantize_rows_fp8():
    x = rng.standard_normal((64, 128)).astype(np.float32)
    x[3] = 0.0
    codes, scale = O.quantize_rows_fp8(x)
    assert codes.dtype == np.uint8 and scale.dtype == np.float32
    assert (codes[3] == 0).all() and scale[3] == 0
    rows = [r for r in range(64) if r != 3]
    # the row's largest magnitude maps to +-448 exactly
    am = np.argmax(np.abs(x[rows]), axis=1)
    assert np.array_equal(codes[rows, am] & 0x7F, np.full(len(rows), 0x7E))
    # dequantised values: within half an E4M3 step of x (relative 1/16 for normals, plus the subnormal quantum)
    deq = O.e4m3_decode(codes) * scale[:, None].astype(np.float64)
    err = np.abs(deq - x)
    assert (err[rows] <= np.abs(x[rows]) / 16 + scale[rows, None] * 2.0 ** -10 + 1e-30).all()
    # codes of the float32 product follow torch's conversion
    inv = (np.float32(448) / np.max(np.abs(x[rows]), axis=1)).astype(np.float32)
    assert np.array_equal(codes[rows], _torch_e4m3((x[rows] * inv[:, None]).astype(np.float32)))


def test_indexer_fp8_reduces_to_plain_indexer():
    # codes of small integers with unit scales: the same scores as the plain indexer on those integers
    ints = np.array([0, 1, 2, 3, 4, 5, 6, 7, 8, 10, 12, 16], dtype=np.float64)
    q = rng.choice(np.concatenate([ints, -ints]), (5, 3, 32))
    k = rng.choice(np.concatenate([ints, -ints]), (40, 32))
    w = rng.uniform(0, 1, (5, 3))
    qc, kc = O.e4m3_encode(q), O.e4m3_encode(k)
    assert np.array_equal(O.e4m3_decode(qc), q) and np.array_equal(O.e4m3_decode(kc), k)
    one_q, one_k = np.ones((5, 3)), np.ones(40)
    I8 = O.indexer_scores_fp8(qc, one_q, w, kc, one_k, pos0=100, m=4)
    assert np.array_equal(I8, O.indexer_scores(q, w, k, pos0=100, m=4))
    # per-key scale multiplies that key's score; per-(query, head) scale weights that head
    ks = rng.uniform(0.5, 2.0, 40)
    qs = rng.uniform(0.5, 2.0, (5, 3))
    I8s = O.indexer_scores_fp8(qc, qs, w, kc, ks, pos0=100, m=4)
    assert np.allclose(I8s, O.indexer_scores(q, w * qs, k, pos0=100, m=4) * ks[None, :], rtol=1e-13, atol=0)


# ---------------------------------------------------------------- FP4 (E2M1) indexer

def test_e2m1_table_ties_and_thresholds():
    vals = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]  # the OCP E2M1 magnitudes, by hand
    assert np.array_equal(O.e2m1_values(), vals)
    assert np.array_equal(O.e2m1_decode(np.arange(16)), vals + [-v for v in vals])
    # every midpoint rounds to the even code
    for y, code in ((0.25, 0), (0.75, 2), (1.25, 2), (1.75, 4), (2.5, 4), (3.5, 6), (5.0, 6)):
        assert O.e2m1_encode(y) == code, y
        assert O.e2m1_encode(-y) == code | 8, y
    assert O.e2m1_encode(7.0) == 7 and O.e2m1_encode(-100.0) == 15 and O.e2m1_encode(-0.0) == 8
    # nearest-value search against a count of the rounding thresholds, on dense values
    y = np.linspace(-8, 8, 64001)
    a = np.abs(y)
    cnt = ((a > 0.25).astype(int) + (a >= 0.75) + (a > 1.25) + (a >= 1.75) + (a > 2.5) + (a >= 3.5) + (a > 5))
    assert np.array_equal(O.e2m1_encode(y) & 7, cnt)


def test_quantize_rows_fp4_and_packing():
    x = rng.standard_normal((40, 64)).astype(np.float32)
    x[5] = 0.0
    codes, scale = O.quantize_rows_fp4(x)
    assert (codes[5] == 0).all() and scale[5] == 0
    rows = [r for r in range(40) if r != 5]
    am = np.argmax(np.abs(x[rows]), axis=1)
    assert np.array_equal(codes[rows, am] & 7, np.full(len(rows), 7))   # the largest magnitude maps to 6
    deq = O.e2m1_decode(codes) * scale[:, None].astype(np.float64)
    assert (np.abs(deq - x)[rows] <= scale[rows, None] * 1.0 + 1e-12).all()  # half of the widest step (4..6)
    packed = O.pack_nibbles(codes)
    assert packed.shape == (40, 32)
    assert np.array_equal(packed & 0xF, codes[:, 0::2]) and np.array_equal(packed >> 4, codes[:, 1::2])


def test_indexer_fp4_reduces_to_plain_indexer():
    v = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6], dtype=np.float64)
    q = rng.choice(np.concatenate([v, -v]), (4, 3, 32))
    k = rng.choice(np.concatenate([v, -v]), (30, 32))
    w = rng.uniform(0, 1, (4, 3))
    qc, kc = O.e2m1_encode(q), O.e2m1_encode(k)
    assert np.array_equal(O.e2m1_decode(qc), q) and np.array_equal(O.e2m1_decode(kc), k)
    I4 = O.indexer_scores_fp4(qc, np.ones((4, 3)), w, kc, np.ones(30), pos0=80, m=4)
    assert np.array_equal(I4, O.indexer_scores(q, w, k, pos0=80, m=4))
    ks = rng.uniform(0.5, 2.0, 30)
    assert np.allclose(O.indexer_scores_fp4(qc, np.ones((4, 3)), w, kc, ks, pos0=80, m=4),
                       O.indexer_scores(q, w, k, pos0=80, m=4) * ks[None, :], rtol=1e-13, atol=0)


# ---------------------------------------------------------------- MX-FP4 (E2M1 + E8M0 block scales) indexer

def test_mxfp4_hand_blocks():
    x = np.zeros((3, 64), dtype=np.float32)
    # block 0: amax 6 = 1.5 * 2**2 -> shared exponent 0 (code 127), values exact or rounded to even
    x[0, :6] = [6.0, -3.0, 0.5, 0.25, 1.25, 5.0]
    # block 1: amax 0.3 -> floor(log2 0.3) = -2 -> exponent -4 (code 123), scale 1/16
    x[0, 32:35] = [0.3, -0.2, 0.01]
    # row 1: block 0 all zero; block 1 amax 1000 -> floor(log2) = 9 -> exponent 7 (code 134)
    x[1, 40:42] = [1000.0, 100.0]
    # row 2: tiny values: amax 2**-130 -> exponent -132 clamps to code 0 (scale 2**-127), values round to 0
    x[2, 0] = 2.0 ** -130
    codes, sc = O.quantize_rows_mxfp4(x)
    assert sc.tolist() == [[127, 123], [0, 134], [0, 0]]
    assert codes[0, :6].tolist() == [7, 8 | 5, 1, 0, 2, 6]     # 0.25 and 1.25 tie to the even code; 5 -> 4
    assert codes[0, 32:35].tolist() == [6, 8 | 5, 0]           # 4.8 -> 4, -3.2 -> -3, 0.16 -> 0
    assert codes[1, 40:42].tolist() == [7, 2]                  # 1000/128 = 7.8 saturates to 6; 100/128 = 0.78 -> 1
    assert (codes[1, :32] == 0).all() and codes[2, 0] == 0
    deq = O.dequantize_mxfp4(codes, sc)
    assert deq[0, :6].tolist() == [6.0, -3.0, 0.5, 0.0, 1.0, 4.0]
    assert deq[0, 32:35].tolist() == [0.25, -0.1875, 0.0]
    assert deq[1, 40:42].tolist() == [768.0, 128.0]


def test_mxfp4_scale_is_the_standard_exponent():
    # over random blocks: the largest magnitude sits in [4, 8) scale units, every value within
    # half of the widest E2M1 step (2 scale units between 4 and 6) or saturated at 6 units
    x = (rng.standard_normal((50, 128)) * np.exp2(rng.integers(-20, 20, (50, 1)))).astype(np.float32)
    codes, sc = O.quantize_rows_mxfp4(x)
    xb = x.reshape(50, 4, 32).astype(np.float64)
    X = np.exp2(sc.astype(np.float64) - 127)
    r = np.abs(xb).max(axis=-1) / X
    assert ((r >= 4) & (r < 8)).all()
    deq = O.dequantize_mxfp4(codes, sc).reshape(50, 4, 32)
    err = np.abs(deq - xb)
    assert (err <= np.maximum(X[..., None], np.abs(xb) - 6 * X[..., None])).all()  # half a 2-unit step, or saturated
    assert (np.abs(deq) <= 6 * X[..., None]).all()


def test_indexer_mxfp4_reduces_to_plain_indexer():
    v = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6], dtype=np.float64)
    q = rng.choice(np.concatenate([v, -v]), (4, 3, 64))
    k = rng.choice(np.concatenate([v, -v]), (30, 64))
    w = rng.uniform(0, 1, (4, 3))
    qc, kc = O.e2m1_encode(q), O.e2m1_encode(k)
    one_q, one_k = np.full((4, 3, 2), 127, np.uint8), np.full((30, 2), 127, np.uint8)
    assert np.array_equal(O.indexer_scores_mxfp4(qc, one_q, w, kc, one_k, pos0=80, m=4),
                          O.indexer_scores(q, w, k, pos0=80, m=4))
    # scaling block 1 of every key by 2**3 is the plain indexer on keys whose second half is 8x
    ks = one_k.copy(); ks[:, 1] = 130
    k2 = k.copy(); k2[:, 32:] *= 8
    assert np.array_equal(O.indexer_scores_mxfp4(qc, one_q, w, kc, ks, pos0=80, m=4),
                          O.indexer_scores(q, w, k2, pos0=80, m=4))


def test_indexer_mxfp8_reduces_to_plain_indexer():
    # small integers are exact E4M3 values; with every scale code 127 (2**0) the MX-FP8 scores are
    # the plain indexer's on those integers, and a scale code of 130 on a block is that block x 8
    ints = np.array([0, 1, 2, 3, 4, 5, 6, 7, 8, 10, 12, 16], dtype=np.float64)
    q = rng.choice(np.concatenate([ints, -ints]), (4, 3, 128))
    k = rng.choice(np.concatenate([ints, -ints]), (30, 128))
    w = rng.uniform(0, 1, (4, 3))
    qc, kc = O.e4m3_encode(q), O.e4m3_encode(k)
    one_q, one_k = np.full((4, 3, 4), 127, np.uint8), np.full((30, 4), 127, np.uint8)
    assert np.array_equal(O.indexer_scores_mxfp8(qc, one_q, w, kc, one_k, pos0=80, m=4),
                          O.indexer_scores(q, w, k, pos0=80, m=4))
    ks = one_k.copy(); ks[:, 2] = 130
    k2 = k.copy(); k2[:, 64:96] *= 8
    assert np.array_equal(O.indexer_scores_mxfp8(qc, one_q, w, kc, ks, pos0=80, m=4),
                          O.indexer_scores(q, w, k2, pos0=80, m=4))
    qs = one_q.copy(); qs[:, :, 0] = 125
    q2 = q.copy(); q2[:, :, :32] /= 4
    assert np.array_equal(O.indexer_scores_mxfp8(qc, qs, w, kc, one_k, pos0=80, m=4),
                          O.indexer_scores(q2, w, k, pos0=80, m=4))


def test_mxfp8_hand_blocks_and_range():
    x = np.zeros((2, 64), dtype=np.float32)
    x[0, :4] = [448.0, -1.0, 300.0, 0.0]     # amax 448 = 1.75 * 2**8 -> shared exponent 0 (code 127)
    x[0, 32:34] = [3.0, 0.001]               # amax 3 -> floor(log2 3) = 1 -> exponent -7 (code 120): 3 -> 384
    x[1, :2] = [1e-3, -5e-4]                 # floor(log2 1e-3) = -10 -> exponent -18 (code 109)
    codes, sc = O.quantize_rows_mxfp8(x)
    assert sc.tolist() == [[127, 120], [109, 0]]
    deq = O.dequantize_mxfp8(codes, sc)
    assert deq[0, :4].tolist() == [448.0, -1.0, 288.0, 0.0]            # 300 -> 288 (E4M3 step 32 there)
    assert deq[0, 32] == 3.0 and deq[0, 33] == 0.0009765625              # 0.128 units -> 0.125 units
    assert abs(deq[1, 0] - 1e-3) <= 2.0 ** -18 * 16 and (deq[1, 32:] == 0).all()
    # random blocks: the largest magnitude lies in [256, 512) scale units, saturating at 448
    xr = (rng.standard_normal((40, 128)) * np.exp2(rng.integers(-20, 20, (40, 1)))).astype(np.float32)
    c, s = O.quantize_rows_mxfp8(xr)
    r = np.abs(xr.reshape(40, 4, 32)).max(axis=-1) / np.exp2(s.astype(np.float64) - 127)
    assert ((r >= 256) & (r < 512)).all()
    d = O.dequantize_mxfp8(c, s).reshape(40, 4, 32)
    X = np.exp2(s.astype(np.float64) - 127)[..., None]
    xb = xr.reshape(40, 4, 32).astype(np.float64)
    assert (np.abs(d - xb) <= np.maximum(16 * X, np.abs(xb) - 448 * X)).all()   # half a 32-unit step, or saturated


# ---------------------------------------------------------------- FP8 + BF16 KV storage

def test_kv_scale_exponent_is_the_smallest_that_fits():
    a = np.concatenate([rng.uniform(0, 1, 2000) * np.exp2(rng.integers(-40, 40, 2000)),
                        448 * np.exp2(np.arange(-10, 10)), 448 * np.exp2(np.arange(-10, 10)) * (1 + 2.0 ** -20)])
    e = O.kv_scale_exponent(a)
    assert (a <= 448 * np.exp2(e.astype(float))).all()            # fits
    assert (a > 448 * np.exp2(e.astype(float) - 1)).all()         # and one power lower does not
    assert O.kv_scale_exponent(0.0) == 0


def test_kv_fp8_roundtrip_and_errors():
    d, r = 512, 64
    x = O.round_bf16(rng.standard_normal((50, d)) * rng.uniform(0.01, 100, (50, 1)))
    x[7] = 0.0
    codes, rope, scale = O.quantize_kv_fp8(x, r)
    assert codes.shape == (50, d - r) and rope.shape == (50, r)
    assert np.array_equal(np.log2(scale), np.round(np.log2(scale)))   # powers of two
    back = O.dequantize_kv_fp8(codes, rope, scale)
    assert np.array_equal(back[:, d - r:], x[:, d - r:])              # RoPE dims kept exactly (bf16 input)
    err = np.abs(back[:, : d - r] - x[:, : d - r])
    # half an E4M3 step: 1/16 relative for normals, 2**-10 * scale in the subnormal range
    assert (err <= np.abs(x[:, : d - r]) / 16 + scale[:, None] * 2.0 ** -10).all()
    assert (codes[7] == 0).all() and scale[7] == 1.0
    # values already on the grid come back exactly
    grid = O.e4m3_decode(rng.integers(0, 126, (5, d - r))) * np.exp2(rng.integers(-5, 5, (5, 1)))
    g = np.concatenate([grid, np.zeros((5, r))], axis=1)
    c2, r2, s2 = O.quantize_kv_fp8(g, r)
    assert np.array_equal(O.dequantize_kv_fp8(c2, r2, s2), g)
    # the RoPE dims are stored in bf16 (8 significant bits): 1 + 2**-10 -> 1, 1 + 3 * 2**-9 -> 1 + 2**-7
    h = np.zeros((1, 32)); h[0, 0] = 1.0; h[0, 16:18] = [1 + 2.0 ** -10, 1 + 3 * 2.0 ** -9]
    _, r3, _ = O.quantize_kv_fp8(h, 16)
    assert r3[0, :2].tolist() == [1.0, 1 + 2.0 ** -7] and (r3[0, 2:] == 0).all()


def test_page_constants_fixture():
    with open(os.path.join(GOLDEN, "page_constants.json")) as f:
        g = json.load(f)
    assert g["csa_ratio_m"]["value"] == 4 and g["hca_ratio_m_prime"]["value"] == 128
    assert g["topk"]["value"] == 1024 and g["window"]["value"] == 128 and g["rope_dims"]["value"] == 64


# ---------------------------------------------------------------- projections

def test_lowrank_proj_brute_force():
    # small integers: every product and sum is exact in fp64, so the triple loop must agree bit for bit
    cq = rng.integers(-4, 5, size=(3, 5)).astype(np.float64)
    W = rng.integers(-4, 5, size=(5, 7)).astype(np.float64)
    ref = [[sum(cq[t, k] * W[k, n] for k in range(5)) for n in range(7)] for t in range(3)]
    assert np.array_equal(O.lowrank_proj(cq, W), np.array(ref))


def test_grouped_out_proj_hand_case():
    # H = 4 heads of d = 1, G = 2 groups of 2 heads, d_g = 1: u[t, g] = o[t, 2g] Wg[g,0] + o[t, 2g+1] Wg[g,1]
    o = np.array([[[1.0], [2.0], [3.0], [4.0]]])
    Wg = np.array([[[10.0], [100.0]], [[1000.0], [10000.0]]])
    u = O.grouped_out_proj_mid(o, Wg)
    assert np.array_equal(u, np.array([[[210.0], [43000.0]]]))
    Wo = np.array([[1.0, 2.0], [3.0, 5.0]])
    y = O.grouped_out_proj(o, Wg, Wo, round_mid=False)
    assert np.array_equal(y, np.array([[210.0 + 3 * 43000.0, 420.0 + 5 * 43000.0]]))


def test_grouped_out_proj_equals_block_diagonal_dense():
    # contiguous head groups with their own weights == one dense product with a block-diagonal
    # weight; catches interleaved grouping, a transposed group weight or a wrong group order
    from scipy.linalg import block_diag
    T, H, d, G, dg = 5, 6, 4, 3, 7
    o = rng.standard_normal((T, H, d))
    Wg = rng.standard_normal((G, (H // G) * d, dg))
    u = O.grouped_out_proj_mid(o, Wg)
    dense = o.reshape(T, H * d) @ block_diag(*[Wg[g] for g in range(G)])
    np.testing.assert_allclose(u.reshape(T, G * dg), dense, rtol=1e-13, atol=1e-13)
    # G = 1 is a plain product
    W1 = rng.standard_normal((1, H * d, dg))
    np.testing.assert_allclose(O.grouped_out_proj_mid(o, W1)[:, 0], o.reshape(T, H * d) @ W1[0], rtol=1e-13)


def test_grouped_out_proj_identity_weights_and_mid_rounding():
    # identity group and output weights return the heads concatenated; the bf16 rounding of the
    # intermediate is exact on bf16 inputs and changes a non-bf16 intermediate
    T, H, d, G = 3, 4, 2, 2
    o = O.round_bf16(rng.standard_normal((T, H, d)))
    n = (H // G) * d
    Wg = np.stack([np.eye(n)] * G)
    y = O.grouped_out_proj(o, Wg, np.eye(G * n))
    assert np.array_equal(y, o.reshape(T, H * d))
    o2 = rng.standard_normal((T, H, d))
    assert not np.array_equal(O.grouped_out_proj(o2, Wg, np.eye(G * n)),
                              O.grouped_out_proj(o2, Wg, np.eye(G * n), round_mid=False))
