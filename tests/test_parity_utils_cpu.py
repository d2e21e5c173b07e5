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
