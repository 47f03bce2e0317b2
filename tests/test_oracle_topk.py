"""Pins of oracle.topk: bf16 rounding, selection by brute force, causal special cases."""
import numpy as np
import pytest
import torch

from oracle import topk as T
from sparse_mask_load_amd import workloads as W


def test_round_to_bf16_matches_torch_conversion():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(20000) * 10.0 ** rng.integers(-6, 6, 20000),
                        np.array([0.0, 1.0, -1.0, 1.00390625, 1.01171875, 3.0e38])])
    x32 = x.astype(np.float32)  # fp32-exact inputs so fp64 -> bf16 equals fp32 -> bf16
    ref = torch.from_numpy(x32).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(T.round_to_bf16(x32.astype(np.float64)), ref)


def _rank_select(imp, i, k, causal):
    """Brute force: a candidate is selected iff fewer than k candidates beat it."""
    cand = list(range(i + 1)) if causal else list(range(len(imp)))
    chosen = []
    for j in cand:
        beaten_by = sum(1 for t in cand if imp[t] > imp[j] or (imp[t] == imp[j] and t < j))
        if beaten_by < k:
            chosen.append((beaten_by, j))
    return [j for _, j in sorted(chosen)]


def test_selection_brute_force_with_ties():
    rng = np.random.default_rng(1)
    for trial in range(30):
        n = int(rng.integers(1, 40))
        imp = rng.integers(-3, 4, size=n).astype(np.float64)  # many exact ties
        i = int(rng.integers(0, n))
        k = int(rng.integers(1, 12))
        for causal in (True, False):
            got = T.select_row(imp, i, k, causal).tolist()
            assert got == _rank_select(imp, i, k, causal)


def _sdpa_causal(q, k, v):
    t = lambda x: torch.from_numpy(np.asarray(x, np.float64))
    return torch.nn.functional.scaled_dot_product_attention(t(q), t(k), t(v), is_causal=True).numpy()


def test_topk_at_least_n_is_causal_attention():
    w = W.make_custom(1, 2, 96, 32, pattern="topk", top_k=200, dtype="bf16", seed=3)
    O, sels, _ = T.dsa(w.q, w.k, w.v, w.wq, w.wk, w.top_k, causal=True)
    ref = _sdpa_causal(w.q, w.k, w.v).reshape(-1, 32)
    assert np.abs(O - ref).max() < 1e-12
    assert [len(s) for s in sels[:5]] == [1, 2, 3, 4, 5]


def test_rows_below_k_take_every_causal_key():
    w = W.make_custom(1, 1, 160, 32, pattern="topk", top_k=64, dtype="bf16", seed=4)
    rows = [(0, 0, i) for i in range(160)]
    O, sels, _ = T.dsa(w.q, w.k, w.v, w.wq, w.wk, 64, causal=True, rows=rows)
    ref = _sdpa_causal(w.q, w.k, w.v)[0, 0]
    assert np.abs(O[:64] - ref[:64]).max() < 1e-12
    assert all(len(s) == 64 for s in sels[64:])
    assert np.abs(O[64:] - ref[64:]).max() > 1e-3  # later rows really are sparse


def test_selection_is_the_top_of_the_importance():
    w = W.make_custom(1, 1, 300, 64, pattern="topk", top_k=32, dtype="bf16", seed=5)
    _, sels, imps = T.dsa(w.q, w.k, w.v, w.wq, w.wk, 32, causal=True, rows=[(0, 0, 299), (0, 0, 150)])
    for sel, imp, i in zip(sels, imps, (299, 150)):
        assert len(set(sel.tolist())) == 32 and sel.max() <= i
        rest = np.setdiff1d(np.arange(i + 1), sel)
        assert imp[sel].min() >= imp[rest].max()


def test_importance_scale_does_not_change_selection():
    w = W.make_custom(1, 1, 200, 32, pattern="topk", top_k=16, dtype="bf16", seed=6)
    rows = [(0, 0, 199), (0, 0, 77)]
    _, s1, _ = T.dsa(w.q, w.k, w.v, w.wq, w.wk, 16, rows=rows)
    _, s2, _ = T.dsa(w.q, w.k, w.v, w.wq * 4.0, w.wk, 16, rows=rows)  # power of two: exact
    assert all(np.array_equal(a, b) for a, b in zip(s1, s2))


def test_projection_rounding_is_bf16():
    w = W.make_custom(1, 1, 64, 32, pattern="topk", top_k=8, dtype="bf16", seed=7)
    qp, kp = T.projections(w.q[0, 0], w.k[0, 0], w.wq, w.wk)
    ref = torch.from_numpy((w.q[0, 0].astype(np.float64) @ w.wq.astype(np.float64))).to(torch.bfloat16)
    # fp64 products of bf16 values are exact, so fp64 -> bf16 equals the library's rounding of them
    assert np.array_equal(qp, ref.to(torch.float64).numpy())


def test_attention_on_indices_matches_dsa():
    w = W.make_custom(1, 2, 128, 32, pattern="topk", top_k=24, dtype="bf16", seed=8)
    O, sels, _ = T.dsa(w.q, w.k, w.v, w.wq, w.wk, 24)
    idx = np.full((1, 2, 128, 24), -1, np.int64)
    cnt = np.zeros((1, 2, 128), np.int64)
    for r, s in enumerate(sels):
        h, i = divmod(r, 128)
        idx[0, h, i, :len(s)] = s
        cnt[0, h, i] = len(s)
    O2 = T.attention_on_indices(w.q, w.k, w.v, idx, cnt)
    assert np.abs(O - O2).max() == 0


def test_dsa_ratio_page_value(golden):
    g = golden("dsa_ratio.txt")
    n, k = int(g["n"]), int(g["k"])
    assert n // k == 256 and abs(n / k - int(g["approx_ratio"])) / 256 < 0.03
