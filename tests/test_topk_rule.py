"""Pins of the top-k acceptance rule (tests/topk_check.py) on the CPU: the oracle's own
selection passes with no swap, near-tie swaps are accepted and counted, and plausible
mistakes (a missing best key, a key outside the causal window, a duplicate, a short list,
a swap far outside the rounding band) are rejected."""
import numpy as np
import pytest

from oracle import topk as T
from tests.topk_check import check_selection, delta_of


def _row(seed=0, n=200, r=32):
    rng = np.random.default_rng(seed)
    qp = T.round_to_bf16(rng.standard_normal(r))
    kp = T.round_to_bf16(rng.standard_normal((n, r)))
    return qp, kp, kp @ qp


def test_oracle_selection_passes_without_swaps():
    qp, kp, imp = _row()
    for i in (0, 5, 63, 64, 150, 199):
        sel = T.select_row(imp, i, 64, True)
        cand = np.arange(i + 1)
        assert check_selection(sel, imp, i, 64, True, delta_of(qp, kp, cand)) == 0


def test_near_tie_swap_is_counted():
    qp, kp, imp = _row(1)
    i, k = 199, 32
    ref = T.select_row(imp, i, k, True)
    order = np.lexsort((np.arange(i + 1), -imp[: i + 1]))
    first_out = order[k]  # best unselected key
    sel = ref.copy()
    sel[-1] = first_out  # swap the k-th for the (k+1)-th
    gap = abs(imp[ref[-1]] - imp[first_out])
    assert check_selection(sel, imp, i, k, True, gap + 1e-12) == 1
    with pytest.raises(AssertionError):
        check_selection(sel, imp, i, k, True, gap / 4)


@pytest.mark.parametrize("mistake", ["drop_best", "outside", "duplicate", "short", "far_swap"])
def test_mistakes_are_rejected(mistake):
    qp, kp, imp = _row(2)
    i, k = 150, 40
    cand = np.arange(i + 1)
    sel = T.select_row(imp, i, k, True).copy()
    d = delta_of(qp, kp, cand)
    order = np.lexsort((cand, -imp[cand]))
    if mistake == "drop_best":
        sel[0] = order[-1]  # replace the best key by the worst candidate
    elif mistake == "outside":
        sel[3] = i + 1  # not causal
    elif mistake == "duplicate":
        sel[3] = sel[4]
    elif mistake == "short":
        sel = sel[:-1]
    else:
        sel[-1] = order[k + 30]  # well below the k-th importance
    with pytest.raises(AssertionError):
        check_selection(sel, imp, i, k, True, d)


def test_short_rows_take_every_candidate():
    qp, kp, imp = _row(3)
    for i in range(10):
        sel = T.select_row(imp, i, 64, True)
        assert sorted(sel) == list(range(i + 1))
        assert check_selection(sel, imp, i, 64, True, 0.0) == 0
