"""CPU checks of the parity helpers themselves: the bounded top-k check must
accept any selection consistent with the error bound and reject one that is
not, so that a GPU test passing through it means something."""
import numpy as np
import pytest

from oracle import cskv_oracle as O
from tests.parity_utils import check_topk_row_bounded, fp8_score_bound

rng = np.random.default_rng(99)


def _case(V=3000, HI=8, dI=64):
    qc, qs = O.quantize_rows_fp8(rng.standard_normal((HI, dI)).astype(np.float32))
    kc, ks = O.quantize_rows_fp8(rng.standard_normal((V, dI)).astype(np.float32))
    w = rng.uniform(0, 1, HI)
    I = O.indexer_scores_fp8(qc[None], qs[None], w[None], kc, ks, pos0=4 * V, m=4)[0]
    return I, fp8_score_bound(qc, qs, w, kc, ks, V)


def test_bound_is_positive_and_small():
    I, B = _case()
    assert (B > 0).all()
    assert (B <= 0.05 * np.abs(I).max()).all()


def test_bounded_check_accepts_perturbed_selections():
    I, B = _case()
    V, k = I.size, 200
    for _ in range(20):
        pert = I + rng.uniform(-1, 1, V) * B                 # any scores the bound allows
        sel = O.topk_row(pert, V, k)
        check_topk_row_bounded(sel, I, B, V, k)


def test_bounded_check_rejects_a_wrong_selection():
    I, B = _case()
    V, k = I.size, 200
    sel = O.topk_row(I, V, k)
    best = int(np.argmax(I))
    worst = int(np.argmin(I))
    bad = np.sort(np.concatenate([sel[sel != best], [worst]]))
    with pytest.raises(AssertionError):
        check_topk_row_bounded(bad, I, B, V, k)
    with pytest.raises(AssertionError):
        check_topk_row_bounded(sel[::-1], I, B, V, k)   # not ascending


def _group_model_dot(dq_row, dk_row, mode):
    """One dot product under the FP8 group model: groups of 8 exact products added on the grid
    2**(E - 13) of the group's largest product, finer bits cut (mode 'zero' or 'floor') or rounded."""
    P = (dk_row * dq_row).reshape(-1, 8)
    tot = 0.0
    for grp in P:
        gm = np.abs(grp).max()
        if gm == 0:
            continue
        _, ex = np.frexp(gm)
        g = np.ldexp(1.0, ex - 14)
        if mode == "zero":
            q = np.trunc(grp / g) * g
        elif mode == "floor":
            q = np.floor(grp / g) * g
        else:
            q = np.round(grp / g) * g
        tot += q.sum()
    return tot


def test_e4m3_product_bound_is_tighter_and_holds_for_the_group_model():
    from oracle import cskv_oracle as O
    from tests.parity_utils import e4m3_group_bound, e4m3_product_bound
    r = np.random.default_rng(3)
    HI, dI, V = 4, 64, 300
    qc, qs = O.quantize_rows_fp8(r.standard_normal((HI, dI)).astype(np.float32))
    kc, ks = O.quantize_rows_fp8(r.standard_normal((V, dI)).astype(np.float32))
    dq, dk = O.e4m3_decode(qc), O.e4m3_decode(kc)
    w = r.uniform(0, 1, HI)
    cheap = e4m3_group_bound(dq, dk, w * qs, ks)
    tight = e4m3_product_bound(dq, dk, w * qs, ks, chunk=37)
    assert (tight <= cheap).all() and np.median(tight / cheap) < 0.1
    exact = np.maximum(dk @ dq.T, 0) @ (w * qs) * ks
    for mode in ("zero", "floor", "round"):
        dots = np.array([[_group_model_dot(dq[h], dk[s], mode) for h in range(HI)] for s in range(V)])
        model = np.maximum(dots, 0) @ (w * qs) * ks
        assert (np.abs(model - exact) <= tight).all(), mode


def test_refine_bound_near_kth_only_tightens_and_keeps_decisions():
    from tests.parity_utils import refine_bound_near_kth, undecided_mask
    r = np.random.default_rng(4)
    V, k = 5000, 100
    s = r.standard_normal(V)
    b = np.full(V, 0.05)
    nb = refine_bound_near_kth(s, b, V, k, lambda ix: np.full(ix.size, 0.001))
    assert (nb <= b).all() and (nb < b).any()
    before, after = undecided_mask(s, b, k), undecided_mask(s, nb, k)
    assert after.sum() < before.sum() and not (after & ~before).any()
