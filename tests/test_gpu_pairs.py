"""GPU parity of Q-block pair work items (sa_problem.q_pairs).

A pair item covers Q-blocks 2p and 2p+1 of one (batch, head) and visits the union of their live
tiles.  The plan's pair loads and every work list must equal the oracle's (``pair_counts`` and
the LPT definitions of ``oracle/plan.py``) bit for bit; the attention outputs (full mode, every
chunk partial, one-chunk calls, the merged output and its lse) must match the oracle's
attention, which does not depend on how rows are grouped into work items.
"""
import numpy as np
import pytest
import torch

from oracle import attention as A
from oracle import plan as P
from sparse_mask_load_amd import binding as bd
from sparse_mask_load_amd import workloads as W
from tests import gpu_util as G
from tests import lazy_rescale as LR

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    bd.lib()  # fails loudly if the library is missing


def _check_pair_plan(w, plan, order):
    info = bd.sparse_attn_plan_info(plan)
    B, H, nQ, C, m = w.B, w.H, w.nQ, w.n_chunks, info["num_bins"]
    nP = (nQ + 1) // 2
    ref = P.pair_counts(w.mask, C, w.layout)
    cnt = P.popcount(w.mask, C, w.layout)
    assert np.array_equal(bd.sparse_attn_plan_copy(plan, bd.SA_PLAN_PAIR_ROW, B * H * nP), ref["row"].reshape(-1))
    assert np.array_equal(bd.sparse_attn_plan_copy(plan, bd.SA_PLAN_PAIR_CROW, B * H * C * nP),
                          ref["crow"].reshape(-1))
    assert np.array_equal(bd.sparse_attn_plan_copy(plan, bd.SA_PLAN_ROW, B * H * nQ), cnt["row"].reshape(-1))
    assert info["n_items"] == B * H * nP
    assert info["total_live"] == cnt["total"] and info["load_sum"] == int(ref["row"].sum())
    lists = [(-1, ref["row"])] + [(c, ref["crow"][:, :, c, :]) for c in range(C)]
    for chunk, loads in lists:
        want = P.plan_items(loads, m, order, groups=info["groups"])
        items = bd.sparse_attn_plan_copy(plan, bd.SA_PLAN_ITEMS, B * H * nP, chunk)
        ptr = bd.sparse_attn_plan_copy(plan, bd.SA_PLAN_BIN_PTR, m + 1, chunk)
        bl = bd.sparse_attn_plan_copy(plan, bd.SA_PLAN_BIN_LOAD, m, chunk)
        assert np.array_equal(items, want["items"]) and np.array_equal(ptr, want["bin_ptr"])
        assert np.array_equal(bl, want["bin_load"])
    assert info["makespan"] == P.plan_items(ref["row"], m, order, groups=info["groups"])["makespan"]
    return info


def _check_partials(w, op, mp, lp, c0, c1, scale=None, tc=False, rows=None):
    """Chunk partials of chunks [c0, c1) against the oracle (every row, or the sampled rows)."""
    idx = tuple(np.array(rows).T) if rows is not None else None
    for i, c in enumerate(range(c0, c1)):
        Oc, Mc, Lc = A.chunk_partial(w.q, w.k, w.v, w.mask, w.block, w.n_chunks, w.layout, c, scale=scale,
                                     token_causal=tc, rows=rows)
        got_m, got_l, got_o = G.to64(mp[i]), G.to64(lp[i]), G.to64(op[i])
        if idx is not None:
            got_m, got_l, got_o = got_m[idx], got_l[idx], got_o[idx]
        assert np.array_equal(np.isneginf(got_m), np.isneginf(Mc)), f"empty-chunk rows differ in chunk {c}"
        fin = np.isfinite(Mc)
        if fin.any():
            G.assert_close(got_m[fin], Mc[fin], (2e-3, 1e-4), f"m chunk {c}")
            G.assert_close(got_l[fin] / Lc[fin], np.ones(fin.sum()), G.ROWSUM_TOL, f"l chunk {c}")
            G.assert_close(got_o[fin] / got_l[fin][..., None], Oc[fin] / Lc[fin][..., None], G.BF16_TOL,
                           f"O/l chunk {c}")
        assert (got_o[~fin] == 0).all() and (got_l[~fin] == 0).all()


def _check_every_row(w, plan, q, k, v, scale=None, tc=False):
    C = w.n_chunks
    ref, ref_lse = A.masked_attention(w.q, w.k, w.v, w.mask, w.block, scale=scale, token_causal=tc)
    o = G.run_full(plan, q, k, v)
    G.assert_close(G.to64(o), ref, G.BF16_TOL, "full")
    op, mp, lp = G.run_partial(plan, q, k, v, 0, C)
    _check_partials(w, op, mp, lp, 0, C, scale, tc)
    om, lse = G.merge(op, mp, lp)
    G.assert_close(G.to64(om), ref, G.BF16_TOL, "merged")
    got_lse = G.to64(lse)
    assert np.array_equal(np.isneginf(got_lse), np.isneginf(ref_lse))
    fin = np.isfinite(ref_lse)
    if fin.any():
        G.assert_close(got_lse[fin], ref_lse[fin], G.ROWSUM_TOL, "lse")
    # one ring step at a time: each chunk's own list
    for c in range(C):
        op1, mp1, lp1 = G.run_partial(plan, q, k, v, c, c + 1)
        _check_partials(w, op1, mp1, lp1, c, c + 1, scale, tc)


PAIR_CASES = [
    # (B, H, S, D, C, pattern, density, token_causal, [B,S,H,D] strides, layout)
    (1, 2, 1024, 128, 4, "causal", 0.0, False, False, "contiguous"),
    (1, 3, 1152, 128, 3, "bernoulli", 0.5, False, False, "contiguous"),  # odd nQ = 9: a lone last row
    (2, 2, 1024, 64, 2, "bernoulli", 0.4, False, True, "contiguous"),   # D 64, [B,S,H,D] strides
    (1, 2, 1024, 128, 4, "causal", 0.0, True, False, "contiguous"),     # token-level causality
    (1, 2, 640, 128, 1, "zipf", 0.5, True, False, "contiguous"),        # token-causal, odd nQ, one chunk
    (1, 2, 768, 128, 3, "zipf", 0.5, False, False, "contiguous"),
    (1, 2, 512, 128, 2, "empty", 0.0, False, False, "contiguous"),
    (1, 2, 2048, 128, 4, "causal", 0.0, False, False, "striped"),      # striped: 32-key groups
    (1, 2, 2048, 128, 2, "bernoulli", 0.5, False, True, "striped"),    # 64-key groups, strides
    (1, 2, 1024, 128, 2, "ones", 0.0, True, False, "striped"),         # striped token-causal
    (1, 3, 1152, 64, 1, "zipf", 0.5, False, False, "striped"),         # one chunk, odd nQ, D 64
]


@pytest.mark.parametrize("n", range(len(PAIR_CASES)),
                         ids=[f"{c[5]}-S{c[2]}-d{c[3]}-C{c[4]}-{c[9][:4]}{'-tc' if c[7] else ''}"
                              f"{'-bshd' if c[8] else ''}" for c in PAIR_CASES])
def test_pair_cases_every_row(n):
    B, H, S, D, C, pattern, dens, tc, bshd, layout = PAIR_CASES[n]
    w = W.make_custom(B, H, S, D, block=128, n_chunks=C, dtype="bf16", pattern=pattern, density=dens,
                      seed=500 + n, layout=layout)
    print(f"pair case {n}: {PAIR_CASES[n]}", flush=True)
    q, k, v = G.upload(w, layout_bshd=bshd)
    for order, bins in (("lpt", 0), ("lpt", 7), ("lpt_device", 0), ("naive", 5)):
        plan = G.plan_block(w, q, order=order, num_bins=bins, token_causal=tc, q_pairs=True)
        _check_pair_plan(w, plan, order)
        if order == "lpt":
            _check_every_row(w, plan, q, k, v, tc=tc)
        else:  # another item order: the same output bits as the LPT plan's
            o_ref = G.run_full(G.plan_block(w, q, token_causal=tc, q_pairs=True), q, k, v)
            assert torch.equal(G.run_full(plan, q, k, v), o_ref)
        plan.close()


@pytest.mark.parametrize("n", [i for i, c in enumerate(LR.RESCALE_CASES) if c[4] == 128 and c[2] % 128 == 0],
                         ids=lambda n: LR.rescale_case_id(LR.RESCALE_CASES[n]))
def test_pair_rescale_every_row(n):
    """Inputs that move the lazy exponent reference inside a chunk (the CPU replay with the pair
    mapping counts the rescales, ``tests/test_rescale_inputs.py``)."""
    w, scale, tc = LR.make_rescale_case(n)
    print(f"pair rescale case {n}: {LR.rescale_case_id(LR.RESCALE_CASES[n])}", flush=True)
    q, k, v = G.upload(w)
    plan = G.plan_block(w, q, token_causal=tc, q_pairs=True, scale=scale or 0.0)
    _check_pair_plan(w, plan, "lpt")
    _check_every_row(w, plan, q, k, v, scale=scale, tc=tc)
    plan.close()


@pytest.fixture(scope="module")
def causal_w():
    return W.make(3)


def test_causal_pairs_bench_path(causal_w):
    """The causal workload with pair items: the device-planned order over the default bins
    (makespan 260 = the bound 66560 / 256), the partial-mode forward over all 4 chunks and the
    merge, against the oracle on sampled rows and every chunk's partial; full mode as well, and
    close to the single-Q-block items' output."""
    w = causal_w
    q, k, v = G.upload(w)
    plan = G.plan_block(w, q, order="lpt_device", q_pairs=True)
    info = _check_pair_plan(w, plan, "lpt_device")
    assert info["makespan"] == info["lower_bound"] == 260
    C = w.n_chunks
    rows = G.sample_rows(w, 128, seed=9)
    idx = tuple(np.array(rows).T)
    ref, ref_lse = A.masked_attention(w.q, w.k, w.v, w.mask, w.block, rows=rows)
    op, mp, lp = G.run_partial(plan, q, k, v, 0, C)
    _check_partials(w, op, mp, lp, 0, C, rows=rows)
    om, lse = G.merge(op, mp, lp)
    G.assert_close(G.to64(om)[idx], ref, G.BF16_TOL, "pairs merged")
    G.assert_close(G.to64(lse)[idx], ref_lse, G.ROWSUM_TOL, "pairs lse")
    del op, mp, lp
    o = G.run_full(plan, q, k, v)
    G.assert_close(G.to64(o)[idx], ref, G.BF16_TOL, "pairs full")
    # one complete pair (256 rows) late in the mask
    blk_rows = [(0, 11, 2 * 50 * 128 + r) for r in range(256)]
    ref_b, _ = A.masked_attention(w.q, w.k, w.v, w.mask, w.block, rows=blk_rows)
    G.assert_close(G.to64(o)[0, 11, 100 * 128:102 * 128], ref_b, G.BF16_TOL, "pair 50")
    o_single = G.run_full(G.plan_block(w, q, order="lpt_device"), q, k, v)
    G.assert_close(G.to64(o), G.to64(o_single), (2e-2, 1e-3), "pairs vs single Q-blocks")


def test_causal_striped_pairs_against_oracle():
    """The causal workload in the striped layout with pair items: the device-planned order, the
    partial-mode forward and the merge against the oracle on sampled rows, every chunk's partial,
    and full mode."""
    w = W.make(3, layout="striped")
    q, k, v = G.upload(w)
    plan = G.plan_block(w, q, order="lpt_device", q_pairs=True)
    info = _check_pair_plan(w, plan, "lpt_device")
    assert info["makespan"] == info["lower_bound"]
    rows = G.sample_rows(w, 96, seed=12)
    idx = tuple(np.array(rows).T)
    ref, ref_lse = A.masked_attention(w.q, w.k, w.v, w.mask, w.block, rows=rows)
    op, mp, lp = G.run_partial(plan, q, k, v, 0, w.n_chunks)
    _check_partials(w, op, mp, lp, 0, w.n_chunks, rows=rows)
    om, lse = G.merge(op, mp, lp)
    G.assert_close(G.to64(om)[idx], ref, G.BF16_TOL, "striped pairs merged")
    G.assert_close(G.to64(lse)[idx], ref_lse, G.ROWSUM_TOL, "striped pairs lse")
    del op, mp, lp
    G.assert_close(G.to64(G.run_full(plan, q, k, v))[idx], ref, G.BF16_TOL, "striped pairs full")


def test_causal_pairs_token_causal(causal_w):
    w = causal_w
    q, k, v = G.upload(w)
    plan = G.plan_block(w, q, order="lpt_device", q_pairs=True, token_causal=True)
    rows = G.sample_rows(w, 96, seed=10)
    idx = tuple(np.array(rows).T)
    ref, _ = A.masked_attention(w.q, w.k, w.v, w.mask, w.block, rows=rows, token_causal=True)
    G.assert_close(G.to64(G.run_full(plan, q, k, v))[idx], ref, G.BF16_TOL, "pairs token-causal full")
    op, mp, lp = G.run_partial(plan, q, k, v, 0, w.n_chunks)
    _check_partials(w, op, mp, lp, 0, w.n_chunks, tc=True, rows=rows)


def test_pair_trace_covers_every_item_once():
    w = W.make_custom(1, 4, 2048, 128, block=128, n_chunks=2, dtype="bf16", pattern="causal", seed=3)
    q, k, v = G.upload(w)
    plan = G.plan_block(w, q, num_bins=64, q_pairs=True)
    info = bd.sparse_attn_plan_info(plan)
    assert info["n_items"] == 4 * 8
    trace = torch.zeros((info["n_items"], 4), dtype=torch.int64, device="cuda")
    G.run_full(plan, q, k, v, trace=trace)
    tr = trace.cpu().numpy()
    items = bd.sparse_attn_plan_copy(plan, bd.SA_PLAN_ITEMS, info["n_items"])
    ptr = bd.sparse_attn_plan_copy(plan, bd.SA_PLAN_BIN_PTR, info["num_bins"] + 1)
    assert np.array_equal(tr[:, 3] & 0xFFFFFFFF, items)
    assert np.array_equal(tr[:, 3] >> 32, np.repeat(np.arange(info["num_bins"]), np.diff(ptr)))
    assert (tr[:, 1] >= tr[:, 0]).all() and (tr[:, 0] > 0).all()


def test_pairs_rejected_outside_their_variants_on_the_gpu():
    w = W.make_custom(1, 2, 1000, 128, block=128, n_chunks=1, dtype="bf16", pattern="ones")
    q, k, v = G.upload(w)
    with pytest.raises(bd.SparseAttnError) as e:  # S not a multiple of 128
        G.plan_block(w, q, q_pairs=True)
    assert e.value.status == bd.SA_ERR_UNSUPPORTED
