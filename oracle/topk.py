"""Oracle: DSA-style indexer, top-k selection and attention over the selected keys.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).  fp64 numpy.

Follows the 6D-parallel notes, section 7.1 (DeepSeek Sparse Attention):

1. indexer: importance of every (query, key) pair from low-rank projections,
   ``I = (Q Wq)(K Wk)^T``; quadratic in the sequence length, but over rank-r
   vectors, so cheap next to the attention it prunes;
2. the ``top_k`` keys of each query by importance (an index array shaped
   [B, H, n, k]);
3. K and V gathered at those indices;
4. ordinary scaled softmax attention of each query over its selected keys.

Readings where the page is silent:

* Scale: standard attention uses ``1/sqrt(d)``; the page's sketch omits it.
* Causal: candidates for query i are keys j <= i; a row with fewer than k
  candidates takes all of them.
* Ties in importance go to the lower key index.
* Precision of the importance: the page calls the scores rough.  A selection
  is an integer decision taken from floating point, so the oracle takes it in
  the precision the GPU declares: the projections ``Q Wq`` and ``K Wk`` are
  rounded to bfloat16 (nearest, ties to even) and the rank-r dot products of
  those bf16 values are taken exactly (in fp64 they are exact).
"""
from __future__ import annotations

import math
from typing import Optional, Sequence, Tuple

import numpy as np


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round fp64 values to the nearest bfloat16 value (8 significant bits, ties to even)."""
    x = np.asarray(x, dtype=np.float64)
    mant, expo = np.frexp(x)  # x = mant * 2**expo, 0.5 <= |mant| < 1
    return np.ldexp(np.rint(mant * 256.0) / 256.0, expo)


def projections(q, k, wq, wk) -> Tuple[np.ndarray, np.ndarray]:
    """Low-rank projections Q' = bf16(Q Wq), K' = bf16(K Wk): [B, H, n, r] each."""
    qp = np.asarray(q, np.float64) @ np.asarray(wq, np.float64)
    kp = np.asarray(k, np.float64) @ np.asarray(wk, np.float64)
    return round_to_bf16(qp), round_to_bf16(kp)


def select_row(imp_row: np.ndarray, i: int, top_k: int, causal: bool) -> np.ndarray:
    """Indices of the top-k candidates of query i, by importance descending then index ascending."""
    n = imp_row.shape[0]
    cand = np.arange(i + 1) if causal else np.arange(n)
    order = np.lexsort((cand, -imp_row[cand]))
    return cand[order[:min(top_k, cand.shape[0])]]


def attend_selected(q_row, k_bh, v_bh, sel: np.ndarray, scale: float) -> np.ndarray:
    """Softmax attention of one query over the selected keys only."""
    if sel.shape[0] == 0:
        return np.zeros(k_bh.shape[-1])
    s = scale * (np.asarray(k_bh, np.float64)[sel] @ np.asarray(q_row, np.float64))
    p = np.exp(s - s.max())
    return (p @ np.asarray(v_bh, np.float64)[sel]) / p.sum()


def dsa(q, k, v, wq, wk, top_k: int, causal: bool = True, scale: Optional[float] = None,
        rows: Optional[Sequence[Tuple[int, int, int]]] = None):
    """Indexer + top-k + attention.

    Returns ``(O, sel, imp)`` for the requested rows (all rows when ``rows`` is
    None): O [R, D] fp64, ``sel`` a list of index arrays, ``imp`` a list of the
    full importance rows (fp64) used for the decision.
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    B, H, n, D = q.shape
    sc = 1.0 / math.sqrt(D) if scale is None else float(scale)
    if rows is None:
        rows = [(b, h, i) for b in range(B) for h in range(H) for i in range(n)]
    qp_cache, kp_cache = {}, {}
    out = np.zeros((len(rows), D))
    sels, imps = [], []
    for r, (b, h, i) in enumerate(rows):
        if (b, h) not in kp_cache:
            qp, kp = projections(q[b, h], k[b, h], wq, wk)
            qp_cache[(b, h)], kp_cache[(b, h)] = qp, kp
        imp = kp_cache[(b, h)] @ qp_cache[(b, h)][i]
        sel = select_row(imp, i, top_k, causal)
        out[r] = attend_selected(q[b, h, i], k[b, h], v[b, h], sel, sc)
        sels.append(sel)
        imps.append(imp)
    return out, sels, imps


def attention_on_indices(q, k, v, idx, count, scale: Optional[float] = None,
                         rows: Optional[Sequence[Tuple[int, int, int]]] = None) -> np.ndarray:
    """Attention of each query over a given key list idx[b, h, i, :count[b, h, i]]."""
    q = np.asarray(q, np.float64)
    B, H, n, D = q.shape
    sc = 1.0 / math.sqrt(D) if scale is None else float(scale)
    if rows is None:
        rows = [(b, h, i) for b in range(B) for h in range(H) for i in range(n)]
    out = np.zeros((len(rows), D))
    for r, (b, h, i) in enumerate(rows):
        sel = np.asarray(idx[b, h, i, :int(count[b, h, i])], dtype=np.int64)
        out[r] = attend_selected(q[b, h, i], k[b, h], v[b, h], sel, sc)
    return out
