"""Acceptance rule for a top-k selection computed in lower precision than the oracle's.

A selection is an integer decision taken from floating point.  The GPU's importance
I = <Q'_i, K'_j> uses bf16 projections and fp32 sums; the oracle's uses the same bf16
rounding of fp64 projections and exact dot products.  The two can order two keys
differently only when their importances are within the rounding error of the GPU's
arithmetic, so a GPU set is accepted for row i when:

* it holds min(top_k, #candidates) distinct candidates (j <= i when causal);
* every selected key has I64 >= tau - delta and every unselected candidate has
  I64 <= tau + delta, tau being the oracle's k-th importance and
  delta = 2^-7 * max_j sum_t |q'_t k'_t| (one bf16 rounding of either factor of every
  product, plus the fp32 sum, stays below this first-order bound).

Keys swapped inside that band are counted as near-tie swaps.
"""
import numpy as np


def delta_of(qp_row: np.ndarray, kp: np.ndarray, cand: np.ndarray) -> float:
    """First-order rounding band of one row: 2^-7 * max over candidates of sum |q'_t k'_t|."""
    if cand.size == 0:
        return 0.0
    return 2.0 ** -7 * float(np.max(np.abs(kp[cand]) @ np.abs(qp_row)))


def check_selection(sel, imp: np.ndarray, i: int, top_k: int, causal: bool, delta: float) -> int:
    """Asserts the acceptance rule for row i; returns the number of near-tie swaps."""
    n = imp.shape[0]
    cand = np.arange(i + 1) if causal else np.arange(n)
    need = min(top_k, cand.size)
    sel = np.asarray(sel, dtype=np.int64)
    assert sel.size == need, (i, sel.size, need)
    assert np.unique(sel).size == need, (i, "duplicate keys")
    assert sel.size == 0 or (sel.min() >= 0 and sel.max() <= cand[-1]), (i, "key outside the candidates")
    if need == cand.size:
        return 0
    order = np.lexsort((cand, -imp[cand]))
    ref = cand[order[:need]]
    tau = imp[ref[-1]]
    assert np.all(imp[sel] >= tau - delta), (i, float(imp[sel].min()), tau, delta)
    unsel = np.setdiff1d(cand, sel)
    assert np.all(imp[unsel] <= tau + delta), (i, float(imp[unsel].max()), tau, delta)
    return int(np.setdiff1d(sel, ref).size)
