"""GPU parity of token-level causality inside live tiles (keys after the query dropped,
positions in the original sequence, also for striped chunks) against the CPU oracle,
through the C ABI: full outputs, every chunk's partial (O, m, l), the merged result and
its lse, within the same tolerances as the block-masked path."""
import numpy as np
import pytest
import torch

from oracle import attention as A
from sparse_mask_load_amd import binding as bd
from sparse_mask_load_amd import workloads as W
from tests import gpu_util as G

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    bd.lib()


CASES = [
    # (B, H, S, D, block, C, dtype, pattern, density, layout)
    (1, 2, 1000, 128, 128, 4, "bf16", "causal", 0.0, "contiguous"),     # ragged diagonal block
    (2, 2, 640, 64, 64, 2, "bf16", "bernoulli", 0.5, "contiguous"),     # tiles above the diagonal
    (1, 2, 1024, 128, 64, 1, "bf16", "ones", 0.0, "contiguous"),
    (1, 2, 2048, 128, 128, 4, "bf16", "causal", 0.0, "striped"),
    (1, 2, 2048, 64, 128, 2, "bf16", "bernoulli", 0.6, "striped"),
    (1, 2, 1024, 64, 64, 2, "bf16", "causal", 0.0, "striped"),
    (1, 3, 700, 64, 64, 1, "f32", "bernoulli", 0.6, "contiguous"),
    (1, 2, 512, 128, 64, 2, "f32", "causal", 0.0, "striped"),
]


@pytest.mark.parametrize("n", range(len(CASES)),
                         ids=[f"{c[7]}-S{c[2]}-d{c[3]}-b{c[4]}-C{c[5]}-{c[6]}-{c[9][:4]}" for c in CASES])
def test_token_causal_every_row(n):
    B, H, S, D, blk, C, dt, pattern, dens, layout = CASES[n]
    w = W.make_custom(B, H, S, D, block=blk, n_chunks=C, dtype=dt, pattern=pattern, density=dens,
                      seed=300 + n, layout=layout)
    if pattern == "bernoulli":
        w.mask[0, 0, 0] = 0
        w.mask[0, 0, 0, 1] = 1  # the first Q-block sees only a later KV block: rows without keys
    tol = G.tol_for(w)
    q, k, v = G.upload(w, layout_bshd=(B == 2))
    ref, ref_lse = A.masked_attention(w.q, w.k, w.v, w.mask, blk, token_causal=True)
    plan = G.plan_block(w, q, token_causal=True)
    o = G.run_full(plan, q, k, v)
    G.assert_close(G.to64(o), ref, tol, "full")
    op, mp, lp = G.run_partial(plan, q, k, v, 0, C)
    for c in range(C):
        Oc, Mc, Lc = A.chunk_partial(w.q, w.k, w.v, w.mask, blk, C, layout, c, token_causal=True)
        got_m = G.to64(mp[c])
        assert np.array_equal(np.isneginf(got_m), np.isneginf(Mc)), f"empty-chunk rows differ in chunk {c}"
        fin = np.isfinite(Mc)
        if fin.any():
            G.assert_close(got_m[fin], Mc[fin], (2e-3, 1e-4), "m")
            G.assert_close(G.to64(lp[c])[fin] / Lc[fin], np.ones(fin.sum()), G.ROWSUM_TOL, "l relative")
            on = G.to64(op[c])[fin] / G.to64(lp[c])[fin][:, None]
            G.assert_close(on, Oc[fin] / Lc[fin][:, None], tol, "O/l")
        assert (G.to64(op[c])[~fin] == 0).all() and (G.to64(lp[c])[~fin] == 0).all()
    om, lse = G.merge(op, mp, lp, out_dtype=dt)
    G.assert_close(G.to64(om), ref, tol, "merged")
    got_lse = G.to64(lse)
    assert np.array_equal(np.isneginf(got_lse), np.isneginf(ref_lse))
    fin = np.isfinite(ref_lse)
    G.assert_close(got_lse[fin], ref_lse[fin], G.ROWSUM_TOL, "lse")


def test_token_causal_changes_only_diagonal_tiles():
    """Against the block-causal result: rows differ (the diagonal tile loses later keys) and
    the first row of every Q-block keeps only earlier blocks plus its own first key."""
    w = W.make_custom(1, 1, 512, 64, block=64, n_chunks=1, dtype="bf16", pattern="causal", seed=3)
    q, k, v = G.upload(w)
    o_blk = G.to64(G.run_full(G.plan_block(w, q), q, k, v))
    o_tok = G.to64(G.run_full(G.plan_block(w, q, token_causal=True), q, k, v))
    assert np.abs(o_tok - o_blk)[0, 0, :63].max() > 2e-2
    # the last row of each block sees exactly the same keys under both rules
    last = np.arange(63, 512, 64)
    assert np.abs(o_tok[0, 0, last] - o_blk[0, 0, last]).max() <= 4e-3
    # row 0 attends key 0 only
    G.assert_close(o_tok[0, 0, 0], G.to64(v)[0, 0, 0], (4e-3, 4e-3), "row 0")


@pytest.mark.parametrize("layout", ["contiguous", "striped"])
def test_token_causal_causal_workload_sampled_rows(layout):
    """The 16-head, 16384-token causal workload at full size: sampled rows, full and chunked."""
    w = W.make(3)
    q, k, v = G.upload(w)
    plan = G.plan_block(w, q, layout=layout, token_causal=True)
    o = G.to64(G.run_full(plan, q, k, v))
    rows = G.sample_rows(w, 96, seed=31)
    rows += [(0, 7, 128 * 50 + r) for r in (0, 1, 63, 64, 127)]
    ref, _ = A.masked_attention(w.q, w.k, w.v, w.mask, w.block, rows=rows, token_causal=True)
    G.assert_close(np.stack([o[b, h, i] for b, h, i in rows]), ref, G.BF16_TOL, f"full {layout}")
    op, mp, lp = G.run_partial(plan, q, k, v, 0, w.n_chunks)
    om, _ = G.merge(op, mp, lp, want_lse=False)
    del op, mp, lp
    om = G.to64(om)
    G.assert_close(np.stack([om[b, h, i] for b, h, i in rows]), ref, G.BF16_TOL, f"merged {layout}")


def test_token_causal_rejected_for_topk_plans():
    w = W.make_custom(1, 1, 64, 128, pattern="topk", top_k=8, seed=10)
    q, k, _ = G.upload(w)
    prob = bd.make_problem(q, 0, 1, "contiguous", token_causal=True)
    wq = torch.from_numpy(np.ascontiguousarray(w.wq)).to("cuda", torch.bfloat16)
    wk = torch.from_numpy(np.ascontiguousarray(w.wk)).to("cuda", torch.bfloat16)
    with pytest.raises(bd.SparseAttnError):
        bd.sparse_attn_plan(prob, "topk", q=q, k=k, wq=wq, wk=wk, rank=w.rank, top_k=8, causal=True)
