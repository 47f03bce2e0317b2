"""GPU parity of the top-k path (indexer + top-k selection, gather attention) against the
CPU oracle, through the C ABI.

The selection is checked row by row with the acceptance rule of tests/topk_check.py
(near-tie swaps within the bf16 rounding band are allowed and counted), and bit-exactly
where the importances are exactly tied (zero indexer weights, repeated keys).  The
attention over the selected keys is checked against the oracle on the GPU's own key lists
and on the oracle's, within max-abs 2e-2 / mean-abs 2e-3.
"""
import numpy as np
import pytest
import torch

from oracle import topk as T
from sparse_mask_load_amd import binding as bd
from sparse_mask_load_amd import workloads as W
from tests import gpu_util as G
from tests.topk_check import check_selection, delta_of

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    bd.lib()


def _plan_topk(w, q, k, top_k=None, causal=None):
    prob = bd.make_problem(q, 0, 1, "contiguous")
    wq = torch.from_numpy(np.ascontiguousarray(w.wq)).to("cuda", torch.bfloat16)
    wk = torch.from_numpy(np.ascontiguousarray(w.wk)).to("cuda", torch.bfloat16)
    plan = bd.sparse_attn_plan(prob, "topk", q=q, k=k, wq=wq, wk=wk, rank=w.rank,
                               top_k=w.top_k if top_k is None else top_k,
                               causal=w.causal if causal is None else causal)
    torch.cuda.synchronize()
    return plan


def _copy_selection(plan, w, top_k):
    n = w.B * w.H * w.S
    idx = bd.sparse_attn_plan_copy(plan, bd.SA_PLAN_TOPK_IDX, n * top_k).reshape(w.B, w.H, w.S, top_k)
    cnt = bd.sparse_attn_plan_copy(plan, bd.SA_PLAN_TOPK_COUNT, n).reshape(w.B, w.H, w.S)
    return idx, cnt


def _check_rows(w, idx, cnt, rows, top_k, causal):
    swaps = 0
    by_head = {}
    for (b, h, i) in rows:
        by_head.setdefault((b, h), []).append(i)
    for (b, h), ii in by_head.items():
        qp, kp = T.projections(w.q[b, h], w.k[b, h], w.wq, w.wk)
        for i in ii:
            imp = kp @ qp[i]
            cand = np.arange(i + 1) if causal else np.arange(w.S)
            sel = idx[b, h, i, :cnt[b, h, i]]
            swaps += check_selection(sel, imp, i, top_k, causal, delta_of(qp[i], kp, cand))
    return swaps


def _attention_checks(w, q, k, v, plan, idx, cnt, rows, top_k, causal):
    o = G.empty_like_qkv(q)
    bd.sparse_attn_fwd(plan, q, k, v, 0, 1, o=o)
    torch.cuda.synchronize()
    got = G.to64(o)
    got_rows = np.stack([got[b, h, i] for (b, h, i) in rows])
    # A6 alone: the oracle's attention over the GPU's own key lists
    ref_own = T.attention_on_indices(w.q, w.k, w.v, idx, cnt, rows=rows)
    G.assert_close(got_rows, ref_own, G.BF16_TOL, "attention on the GPU's key lists")
    # A5 + A6: the oracle's selection and attention
    ref, _, _ = T.dsa(w.q, w.k, w.v, w.wq, w.wk, top_k, causal=causal, rows=rows)
    G.assert_close(got_rows, ref, G.BF16_TOL, "attention on the oracle's key lists")


CASES = [
    # (B, H, S, top_k, causal, seed): every row fits the candidate buffer / threshold search /
    # non-causal / ragged length (not a multiple of 32) / top_k above most rows' candidates
    (1, 2, 300, 64, True, 0),
    (1, 2, 1500, 512, True, 1),
    (2, 1, 2100, 128, False, 2),
    (1, 1, 777, 512, True, 3),
    (1, 2, 2600, 16, True, 4),
    (1, 1, 40, 512, False, 5),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "B{}H{}S{}k{}{}".format(c[0], c[1], c[2], c[3],
                                                                             "c" if c[4] else "n"))
def test_topk_small_all_rows(case):
    B, H, S, top_k, causal, seed = case
    w = W.make_custom(B, H, S, 128, pattern="topk", top_k=top_k, causal=causal, seed=seed)
    q, k, v = G.upload(w)
    plan = _plan_topk(w, q, k)
    idx, cnt = _copy_selection(plan, w, top_k)
    rows = [(b, h, i) for b in range(B) for h in range(H) for i in range(S)]
    swaps = _check_rows(w, idx, cnt, rows, top_k, causal)
    print(f"near-tie swaps: {swaps} over {len(rows)} rows")
    sample = G.sample_rows(w, 48, seed=seed)
    _attention_checks(w, q, k, v, plan, idx, cnt, sample, top_k, causal)
    info = bd.sparse_attn_plan_info(plan)
    assert info["total_live"] == int(cnt.sum())


def test_topk_d64_strided_layout():
    w = W.make_custom(1, 3, 1200, 64, pattern="topk", top_k=200, causal=True, seed=7)
    q, k, v = G.upload(w, layout_bshd=True)
    plan = _plan_topk(w, q, k)
    idx, cnt = _copy_selection(plan, w, w.top_k)
    rows = [(0, h, i) for h in range(w.H) for i in range(w.S)]
    _check_rows(w, idx, cnt, rows, w.top_k, True)
    _attention_checks(w, q, k, v, plan, idx, cnt, G.sample_rows(w, 32, seed=7), w.top_k, True)


def test_topk_wide_row_stride():
    # rows 2^21 elements apart (a head spans more than 2 GiB of address range): the gather takes
    # its 64-bit row addresses instead of 32-bit offsets from the head's base
    w = W.make_custom(1, 1, 100, 128, pattern="topk", top_k=32, causal=True, seed=8)
    ss = 1 << 21

    def wide(x):
        buf = torch.empty((w.S - 1) * ss + w.D, dtype=torch.bfloat16, device="cuda")
        view = buf.as_strided((1, 1, w.S, w.D), (w.S * ss, w.S * ss, ss, 1))
        view.copy_(torch.from_numpy(np.ascontiguousarray(x)).to("cuda", torch.bfloat16))
        return view
    q, k, v = wide(w.q), wide(w.k), wide(w.v)
    plan = _plan_topk(w, q, k)
    idx, cnt = _copy_selection(plan, w, w.top_k)
    rows = [(0, 0, i) for i in range(w.S)]
    _check_rows(w, idx, cnt, rows, w.top_k, True)
    _attention_checks(w, q, k, v, plan, idx, cnt, rows, w.top_k, True)


def test_topk_all_tied_takes_lowest_indices():
    """Zero indexer weights: every importance is 0, so each row keeps its lowest indices."""
    w = W.make_custom(1, 2, 1100, 128, pattern="topk", top_k=100, causal=True, seed=8)
    w.wq = np.zeros_like(w.wq)
    q, k, v = G.upload(w)
    plan = _plan_topk(w, q, k)
    idx, cnt = _copy_selection(plan, w, w.top_k)
    for h in range(w.H):
        for i in range(w.S):
            need = min(w.top_k, i + 1)
            assert cnt[0, h, i] == need
            assert np.array_equal(np.sort(idx[0, h, i, :need]), np.arange(need)), (h, i)


def test_topk_repeated_keys_tie_break():
    """Keys repeat 7 distinct rows, so importances tie exactly in groups; the lower index wins."""
    w = W.make_custom(1, 1, 900, 128, pattern="topk", top_k=50, causal=False, seed=9)
    w.k[0, 0] = w.k[0, 0, np.arange(w.S) % 7]
    q, k, v = G.upload(w)
    plan = _plan_topk(w, q, k)
    idx, cnt = _copy_selection(plan, w, w.top_k)
    qp, kp = T.projections(w.q[0, 0], w.k[0, 0], w.wq, w.wk)
    for i in range(w.S):
        ref = T.select_row(kp @ qp[i], i, w.top_k, False)
        assert np.array_equal(np.sort(idx[0, 0, i, :cnt[0, 0, i]]), np.sort(ref)), i


def test_topk_argument_errors():
    w = W.make_custom(1, 1, 64, 128, pattern="topk", top_k=8, seed=10)
    q, k, _ = G.upload(w)
    with pytest.raises(bd.SparseAttnError):
        _plan_topk(w, q, k, top_k=513)


def test_topk_workload5_sampled_rows():
    """The 16-head, 32768-token workload at full size; selection and attention on sampled rows."""
    w = W.make(5)
    q, k, v = G.upload(w)
    plan = _plan_topk(w, q, k)
    idx, cnt = _copy_selection(plan, w, w.top_k)
    need = np.minimum(w.top_k, np.arange(w.S) + 1)
    assert np.array_equal(cnt, np.broadcast_to(need, cnt.shape))
    rng = np.random.default_rng(5)
    rows = {(0, h, i) for h in (0, 7, 15) for i in (0, 1, 511, 512, 703, 704, 705, 2047, 2048, 32767)}
    while len(rows) < 64:
        rows.add((0, int(rng.integers(0, w.H)), int(rng.integers(0, w.S))))
    rows = sorted(rows)
    swaps = _check_rows(w, idx, cnt, rows, w.top_k, True)
    print(f"near-tie swaps: {swaps} over {len(rows)} sampled rows")
    _attention_checks(w, q, k, v, plan, idx, cnt, rows[:24], w.top_k, True)
