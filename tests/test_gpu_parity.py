"""GPU parity of the block-sparse path (popcount, LPT plan, attention, chunk merge) against
the CPU oracle, through the C ABI.  Integer results are compared bit-exactly; attention
outputs within max-abs 2e-2 / mean-abs 2e-3 (bf16) or 1e-4 (fp32)."""
import numpy as np
import pytest
import torch

from oracle import attention as A
from oracle import plan as P
from sparse_mask_load_amd import binding as bd
from sparse_mask_load_amd import workloads as W
from tests import gpu_util as G

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    bd.lib()  # fails loudly if the library is missing


def _check_plan(w, plan, order, layout=None):
    layout = layout or w.layout
    info = bd.sparse_attn_plan_info(plan)
    B, H, nQ, C, m = w.B, w.H, w.nQ, w.n_chunks, info["num_bins"]
    ref = P.popcount(w.mask, C, layout)
    row = bd.sparse_attn_plan_copy(plan, bd.SA_PLAN_ROW, B * H * nQ)
    col = bd.sparse_attn_plan_copy(plan, bd.SA_PLAN_COL, B * H * nQ)
    crow = bd.sparse_attn_plan_copy(plan, bd.SA_PLAN_CROW, B * H * C * nQ)
    assert np.array_equal(row, ref["row"].reshape(-1))
    assert np.array_equal(col, ref["col"].reshape(-1))
    assert np.array_equal(crow, ref["crow"].reshape(-1))
    assert info["total_live"] == ref["total"]
    lists = [(-1, ref["row"])] + [(c, ref["crow"][:, :, c, :]) for c in range(C)]
    for chunk, loads in lists:
        want = P.plan_items(loads, m, order, groups=info["groups"])
        items = bd.sparse_attn_plan_copy(plan, bd.SA_PLAN_ITEMS, B * H * nQ, chunk)
        ptr = bd.sparse_attn_plan_copy(plan, bd.SA_PLAN_BIN_PTR, m + 1, chunk)
        bl = bd.sparse_attn_plan_copy(plan, bd.SA_PLAN_BIN_LOAD, m, chunk)
        assert np.array_equal(items, want["items"]) and np.array_equal(ptr, want["bin_ptr"])
        assert np.array_equal(bl, want["bin_load"])
    assert info["makespan"] == P.plan_items(ref["row"], m, order, groups=info["groups"])["makespan"]
    return info


def _full_oracle(w):
    O, _ = A.masked_attention(w.q, w.k, w.v, w.mask, w.block)
    return O


# ---------------------------------------------------------------- workload 1: tiny fp32

@pytest.mark.parametrize("order", ["lpt", "naive"])
def test_tiny_f32_full_partial_merge(order):
    w = W.make(1)
    q, k, v = G.upload(w)
    plan = G.plan_block(w, q, order=order, num_bins=2)
    _check_plan(w, plan, order)
    ref = _full_oracle(w)
    o = G.run_full(plan, q, k, v)
    G.assert_close(G.to64(o), ref, G.F32_TOL, "tiny full")
    op, mp, lp = G.run_partial(plan, q, k, v, 0, w.n_chunks)
    for c in range(w.n_chunks):
        Oc, Mc, Lc = A.chunk_partial(w.q, w.k, w.v, w.mask, w.block, w.n_chunks, w.layout, c)
        assert np.array_equal(np.isneginf(G.to64(mp[c])), np.isneginf(Mc))
        fin = np.isfinite(Mc)
        G.assert_close(G.to64(mp[c])[fin], Mc[fin], (1e-5, 1e-5), "m")
        G.assert_close(G.to64(lp[c]), Lc, (1e-4, 1e-5), "l")
        G.assert_close(G.to64(op[c]), Oc, (1e-4, 1e-5), "O")
    om, lse = G.merge(op, mp, lp, out_dtype="f32")
    G.assert_close(G.to64(om), ref, G.F32_TOL, "tiny merged")


# ---------------------------------------------------------------- workload 2: video-like

def test_video_bf16_full_and_chunked():
    w = W.make(2)
    q, k, v = G.upload(w)
    plan = G.plan_block(w, q)
    _check_plan(w, plan, "lpt")
    ref = _full_oracle(w)
    o = G.run_full(plan, q, k, v)
    G.assert_close(G.to64(o), ref, G.BF16_TOL, "video full")
    op, mp, lp = G.run_partial(plan, q, k, v, 0, w.n_chunks)
    om, lse = G.merge(op, mp, lp)
    G.assert_close(G.to64(om), ref, G.BF16_TOL, "video merged")
    # one ring step at a time (per-chunk work lists) equals the single chunked launch
    for c in range(w.n_chunks):
        o1, m1, l1 = G.run_partial(plan, q, k, v, c, c + 1)
        assert torch.equal(m1[0], mp[c]) and torch.equal(l1[0], lp[c]) and torch.equal(o1[0], op[c])


# ---------------------------------------------------------------- workload 3: causal long sequence

@pytest.fixture(scope="module")
def causal_w():
    return W.make(3)


def test_causal_plan_and_balance(causal_w):
    w = causal_w
    q, k, v = G.upload(w)
    for order in ("lpt", "naive"):
        plan = G.plan_block(w, q, order=order, num_bins=256)
        info = _check_plan(w, plan, order)
        if order == "lpt":
            assert info["makespan"] == info["lower_bound"] == 516
        else:
            assert info["makespan"] / (info["total_live"] / 256) > 1.9


@pytest.mark.parametrize("layout", ["contiguous", "striped"])
def test_causal_full_sampled_rows(causal_w, layout):
    w = causal_w
    q, k, v = G.upload(w)
    plan = G.plan_block(w, q, layout=layout)
    _check_plan(w, plan, "lpt", layout)
    o = G.to64(G.run_full(plan, q, k, v))
    rows = G.sample_rows(w, 128, seed=3)
    ref, _ = A.masked_attention(w.q, w.k, w.v, w.mask, w.block, rows=rows)
    got = np.stack([o[b, h, i] for b, h, i in rows])
    G.assert_close(got, ref, G.BF16_TOL, f"causal {layout}")
    # one complete Q-block (all 128 rows) in a late row of the mask
    blk_rows = [(0, 5, 100 * 128 + r) for r in range(128)]
    ref_b, _ = A.masked_attention(w.q, w.k, w.v, w.mask, w.block, rows=blk_rows)
    G.assert_close(o[0, 5, 100 * 128:101 * 128], ref_b, G.BF16_TOL, "causal block 100")


def test_causal_striped_equals_contiguous_and_chunked(causal_w):
    w = causal_w
    q, k, v = G.upload(w)
    pc = G.plan_block(w, q, layout="contiguous")
    ps = G.plan_block(w, q, layout="striped")
    oc = G.run_full(pc, q, k, v)
    os_ = G.run_full(ps, q, k, v)
    G.assert_close(G.to64(os_), G.to64(oc), (2e-2, 1e-3), "striped vs contiguous")
    for plan, name in ((pc, "contiguous"), (ps, "striped")):
        op, mp, lp = G.run_partial(plan, q, k, v, 0, w.n_chunks)
        om, _ = G.merge(op, mp, lp)
        G.assert_close(G.to64(om), G.to64(oc), (2e-2, 1e-3), f"merged {name}")
        del op, mp, lp


def test_causal_bench_path_against_oracle(causal_w):
    """bench.py's step exactly: the device-planned LPT order over the default bins, the
    partial-mode forward over all 4 chunks, then chunk_merge.  Sampled rows of the merged output
    and lse, and of every chunk partial (m, l, O / l), are compared with the oracle directly."""
    w = causal_w
    q, k, v = G.upload(w)
    plan = G.plan_block(w, q, order="lpt_device")
    C = w.n_chunks
    op, mp, lp = G.run_partial(plan, q, k, v, 0, C)
    om, lse = G.merge(op, mp, lp)
    rows = G.sample_rows(w, 128, seed=7)
    idx = tuple(np.array(rows).T)
    ref, ref_lse = A.masked_attention(w.q, w.k, w.v, w.mask, w.block, rows=rows)
    G.assert_close(G.to64(om)[idx], ref, G.BF16_TOL, "bench path merged")
    G.assert_close(G.to64(lse)[idx], ref_lse, G.ROWSUM_TOL, "bench path lse")
    for c in range(C):
        Oc, Mc, Lc = A.chunk_partial(w.q, w.k, w.v, w.mask, w.block, C, w.layout, c, rows=rows)
        got_m, got_l, got_o = G.to64(mp[c])[idx], G.to64(lp[c])[idx], G.to64(op[c])[idx]
        assert np.array_equal(np.isneginf(got_m), np.isneginf(Mc))
        fin = np.isfinite(Mc)
        G.assert_close(got_m[fin], Mc[fin], (2e-3, 1e-4), f"m chunk {c}")
        G.assert_close(got_l[fin] / Lc[fin], np.ones(fin.sum()), G.ROWSUM_TOL, f"l chunk {c}")
        G.assert_close(got_o[fin] / got_l[fin][:, None], Oc[fin] / Lc[fin][:, None], G.BF16_TOL, f"O/l chunk {c}")
        assert (got_o[~fin] == 0).all() and (got_l[~fin] == 0).all()
    del op, mp, lp


# ---------------------------------------------------------------- workload 4: skewed video

def test_skewed_plan_full_and_chunked():
    w = W.make(4)
    q, k, v = G.upload(w)
    pn = G.plan_block(w, q, order="naive", num_bins=256)
    _check_plan(w, pn, "naive")
    pl = G.plan_block(w, q, order="lpt", num_bins=256)
    info = _check_plan(w, pl, "lpt")
    assert info["makespan"] <= bd.sparse_attn_plan_info(pn)["makespan"]
    rows = G.sample_rows(w, 96, seed=4)
    ref, _ = A.masked_attention(w.q, w.k, w.v, w.mask, w.block, rows=rows)
    o = G.to64(G.run_full(pl, q, k, v))
    G.assert_close(np.stack([o[b, h, i] for b, h, i in rows]), ref, G.BF16_TOL, "skewed full")
    o_naive = G.to64(G.run_full(pn, q, k, v))
    assert np.array_equal(o_naive, o)  # the order of items does not change any output bit
    op, mp, lp = G.run_partial(pl, q, k, v, 0, w.n_chunks)
    om, _ = G.merge(op, mp, lp)
    om = G.to64(om)
    G.assert_close(np.stack([om[b, h, i] for b, h, i in rows]), ref, G.BF16_TOL, "skewed merged")


# ---------------------------------------------------------------- smaller cases: every tile of the oracle

CASES = [
    # (B, H, S, D, block, C, dtype, pattern, density, layout)
    (1, 3, 1000, 128, 128, 1, "bf16", "bernoulli", 0.5, "contiguous"),   # ragged last block
    (2, 2, 640, 64, 64, 2, "bf16", "bernoulli", 0.4, "contiguous"),
    (1, 2, 1000, 64, 64, 4, "bf16", "zipf", 0.4, "contiguous"),         # ragged, 4 chunks
    (1, 2, 1024, 128, 64, 4, "bf16", "causal", 0.0, "contiguous"),
    (1, 2, 1024, 64, 128, 2, "bf16", "bernoulli", 0.3, "contiguous"),
    (1, 2, 2048, 128, 128, 4, "bf16", "causal", 0.0, "striped"),
    (1, 2, 2048, 128, 128, 2, "bf16", "bernoulli", 0.5, "striped"),
    (1, 2, 512, 64, 64, 2, "bf16", "bernoulli", 0.5, "striped"),
    (1, 3, 700, 64, 64, 1, "f32", "bernoulli", 0.5, "contiguous"),      # ragged fp32
    (1, 2, 768, 128, 64, 3, "f32", "zipf", 0.5, "contiguous"),
    (1, 2, 512, 128, 64, 2, "f32", "causal", 0.0, "striped"),
    (1, 2, 384, 128, 128, 3, "bf16", "empty", 0.0, "contiguous"),
]


@pytest.mark.parametrize("n", range(len(CASES)),
                         ids=[f"{c[7]}-S{c[2]}-d{c[3]}-b{c[4]}-C{c[5]}-{c[6]}-{c[9][:4]}" for c in CASES])
def test_small_cases_every_row(n):
    B, H, S, D, blk, C, dt, pattern, dens, layout = CASES[n]
    w = W.make_custom(B, H, S, D, block=blk, n_chunks=C, dtype=dt, pattern=pattern, density=dens,
                      seed=100 + n, layout=layout)
    tol = G.tol_for(w)
    q, k, v = G.upload(w, layout_bshd=(B == 2))
    for bins in (0, 7):
        plan = G.plan_block(w, q, num_bins=bins)
        _check_plan(w, plan, "lpt")
        ref = _full_oracle(w)
        o = G.run_full(plan, q, k, v)
        G.assert_close(G.to64(o), ref, tol, "full")
        op, mp, lp = G.run_partial(plan, q, k, v, 0, C)
        for c in range(C):
            Oc, Mc, Lc = A.chunk_partial(w.q, w.k, w.v, w.mask, blk, C, layout, c)
            got_m = G.to64(mp[c])
            assert np.array_equal(np.isneginf(got_m), np.isneginf(Mc)), "empty-chunk rows differ"
            fin = np.isfinite(Mc)
            if fin.any():
                G.assert_close(got_m[fin], Mc[fin], (2e-3, 1e-4), "m")
                G.assert_close(G.to64(lp[c])[fin] / Lc[fin], np.ones(fin.sum()), G.ROWSUM_TOL, "l relative")
                on = G.to64(op[c])[fin] / G.to64(lp[c])[fin][:, None]
                G.assert_close(on, Oc[fin] / Lc[fin][:, None], tol, "O/l")
            assert (G.to64(op[c])[~fin] == 0).all() and (G.to64(lp[c])[~fin] == 0).all()
        om, lse = G.merge(op, mp, lp, out_dtype=dt)
        G.assert_close(G.to64(om), ref, tol, "merged")
        _, ref_lse = A.masked_attention(w.q, w.k, w.v, w.mask, blk)
        got_lse = G.to64(lse)
        assert np.array_equal(np.isneginf(got_lse), np.isneginf(ref_lse))
        fin = np.isfinite(ref_lse)
        if fin.any():
            G.assert_close(got_lse[fin], ref_lse[fin], G.ROWSUM_TOL, "lse")
        del plan


def test_mask_sensitivity_on_gpu():
    w = W.make_custom(1, 1, 512, 64, block=64, n_chunks=1, dtype="bf16", pattern="ones", seed=2)
    q, k, v = G.upload(w)
    o1 = G.to64(G.run_full(G.plan_block(w, q), q, k, v))
    w.mask[0, 0, 3, 5] = 0
    o2 = G.to64(G.run_full(G.plan_block(w, q), q, k, v))
    diff = np.abs(o2 - o1)
    assert diff[0, 0, 192:256].max() > 2e-2
    assert diff[0, 0, :192].max() == 0 and diff[0, 0, 256:].max() == 0


def test_chunk_merge_against_oracle_with_empty_parts():
    rng = np.random.default_rng(5)
    n, rows, D = 5, 3000, 128
    O = rng.standard_normal((n, rows, D)).astype(np.float32)
    M = rng.standard_normal((n, rows)).astype(np.float32) * 3
    L = rng.uniform(0.5, 20, (n, rows)).astype(np.float32)
    M[1, ::3] = -np.inf
    L[1, ::3] = 0
    O[1, ::3] = 0
    M[:, 7] = -np.inf
    L[:, 7] = 0
    O[:, 7] = 0
    ref, ref_lse = A.merge([(O[i], M[i], L[i]) for i in range(n)])
    op = torch.from_numpy(O).cuda()
    mp = torch.from_numpy(M).cuda()
    lp = torch.from_numpy(L).cuda()
    for out_dtype, tol in (("f32", (1e-5, 1e-6)), ("bf16", G.BF16_TOL)):
        out = torch.empty((rows, D), dtype=torch.float32 if out_dtype == "f32" else torch.bfloat16, device="cuda")
        lse = torch.empty(rows, dtype=torch.float32, device="cuda")
        bd.chunk_merge([op[i] for i in range(n)], [mp[i] for i in range(n)], [lp[i] for i in range(n)], rows, D,
                       out, out_dtype, lse)
        torch.cuda.synchronize()
        G.assert_close(G.to64(out), ref, tol, f"merge {out_dtype}")
        got_lse = G.to64(lse)
        assert np.isneginf(got_lse[7]) and (G.to64(out)[7] == 0).all()
        fin = np.isfinite(ref_lse)
        G.assert_close(got_lse[fin], ref_lse[fin], (1e-5, 1e-6), "merge lse")


@pytest.mark.parametrize("n", [1, 2, 3, 4, 7, 9, 64])
@pytest.mark.parametrize("D", [64, 128])
def test_chunk_merge_part_counts(n, D):
    """Part counts around the merge's groups of four reads (and the 64-part limit), with empty parts anywhere."""
    rng = np.random.default_rng(100 + n + D)
    rows = 777
    O = rng.standard_normal((n, rows, D)).astype(np.float32)
    M = (rng.standard_normal((n, rows)) * 4).astype(np.float32)
    L = rng.uniform(0.25, 50, (n, rows)).astype(np.float32)
    empty = rng.random((n, rows)) < 0.3
    empty[:, 11] = True  # a row without any key
    empty[0, 12] = True  # first part empty
    empty[-1, 13] = True  # last part empty
    M[empty] = -np.inf
    L[empty] = 0
    O[empty] = 0
    ref, ref_lse = A.merge([(O[i], M[i], L[i]) for i in range(n)])
    op, mp, lp = (torch.from_numpy(x).cuda() for x in (O, M, L))
    out = torch.empty((rows, D), dtype=torch.float32, device="cuda")
    lse = torch.empty(rows, dtype=torch.float32, device="cuda")
    bd.chunk_merge([op[i] for i in range(n)], [mp[i] for i in range(n)], [lp[i] for i in range(n)], rows, D,
                   out, "f32", lse)
    torch.cuda.synchronize()
    G.assert_close(G.to64(out), ref, (1e-5, 1e-6), f"merge n={n} D={D}")
    got_lse = G.to64(lse)
    assert np.isneginf(got_lse[11]) and (G.to64(out)[11] == 0).all()
    fin = np.isfinite(ref_lse)
    assert np.array_equal(np.isfinite(got_lse), fin)
    G.assert_close(got_lse[fin], ref_lse[fin], (1e-5, 1e-6), "merge lse")


def test_trace_covers_every_item_once():
    w = W.make_custom(1, 4, 2048, 128, block=128, n_chunks=2, dtype="bf16", pattern="zipf", density=0.4, seed=3)
    q, k, v = G.upload(w)
    plan = G.plan_block(w, q, num_bins=64)
    info = bd.sparse_attn_plan_info(plan)
    trace = torch.zeros((info["n_items"], 4), dtype=torch.int64, device="cuda")
    G.run_full(plan, q, k, v, trace=trace)
    tr = trace.cpu().numpy()
    items = bd.sparse_attn_plan_copy(plan, bd.SA_PLAN_ITEMS, info["n_items"])
    ptr = bd.sparse_attn_plan_copy(plan, bd.SA_PLAN_BIN_PTR, info["num_bins"] + 1)
    assert np.array_equal(tr[:, 3] & 0xFFFFFFFF, items)
    bins = np.repeat(np.arange(info["num_bins"]), np.diff(ptr))
    assert np.array_equal(tr[:, 3] >> 32, bins)
    assert (tr[:, 1] >= tr[:, 0]).all() and (tr[:, 0] > 0).all()


def test_fwd_argument_errors_on_gpu():
    w = W.make_custom(1, 1, 256, 64, block=64, n_chunks=2, dtype="bf16", pattern="ones")
    q, k, v = G.upload(w)
    plan = G.plan_block(w, q)
    with pytest.raises(bd.SparseAttnError) as e:
        bd.sparse_attn_fwd(plan, q, k, v, 1, 3, o=G.empty_like_qkv(q))
    assert e.value.status == bd.SA_ERR_INVALID
    with pytest.raises(bd.SparseAttnError) as e:
        bd.sparse_attn_fwd(plan, q, k, v, 0, 2, o=None, o_part=torch.empty(1, device="cuda"))
    assert e.value.status == bd.SA_ERR_INVALID


def test_plan_on_side_stream():
    """A plan built on another stream: the forward call on the main stream waits for its lists."""
    w = W.make_custom(1, 2, 512, 128, block=128, n_chunks=2, pattern="bernoulli", density=0.6, seed=21)
    q, k, v = G.upload(w)
    side = torch.cuda.Stream()
    mask = torch.from_numpy(np.ascontiguousarray(w.mask)).cuda()
    torch.cuda.synchronize()
    plan = bd.sparse_attn_plan(bd.make_problem(q, w.block, w.n_chunks, w.layout), "block", mask=mask, stream=side)
    o = G.empty_like_qkv(q)
    bd.sparse_attn_fwd(plan, q, k, v, 0, w.n_chunks, o=o)  # current stream
    torch.cuda.synchronize()
    G.assert_close(G.to64(o), _full_oracle(w), G.tol_for(w), "side-stream plan")


@pytest.mark.parametrize("cfg", [3, 4])
def test_xcd_order_plan_and_output(cfg):
    """Two-level (XCD-affine) LPT plan: bit-exact lists against the oracle with the device's XCD
    count, and the same attention output as the plain LPT order on sampled rows."""
    w = W.make(cfg)
    q, k, v = G.upload(w)
    plan = G.plan_block(w, q, order="lpt_xcd")
    info = _check_plan(w, plan, "lpt_xcd")
    assert info["groups"] >= 1
    o = G.run_full(plan, q, k, v)
    plan2 = G.plan_block(w, q, order="lpt")
    o2 = G.run_full(plan2, q, k, v)
    # the order changes which workgroup runs an item, not the arithmetic of the item
    assert torch.equal(o, o2)


def test_plan_buffers_reused_only_after_their_last_use():
    """A destroyed plan's buffers return to the library's cache while its forward call may still
    be running; the next plan (same sizes, a different mask, on another stream) takes them over
    ordered after that call.  Both outputs must match the oracle."""
    w = W.make(3)
    q, k, v = G.upload(w)
    o1 = G.empty_like_qkv(q)
    plan1 = G.plan_block(w, q, order="lpt_device")
    torch.cuda.synchronize()
    for _ in range(3):  # a queue of work that keeps plan 1's buffers in use for a while
        bd.sparse_attn_fwd(plan1, q, k, v, 0, w.n_chunks, o=o1)
    plan1.close()  # returns at once; the kernels above still read the plan's lists
    w2 = W.make_custom(w.B, w.H, w.S, w.D, block=w.block, n_chunks=w.n_chunks, pattern="bernoulli", density=0.3,
                       seed=77, mask_only=True)
    w2.q, w2.k, w2.v = w.q, w.k, w.v
    side = torch.cuda.Stream()
    mask2 = torch.from_numpy(np.ascontiguousarray(w2.mask)).cuda()
    plan2 = bd.sparse_attn_plan(bd.make_problem(q, w.block, w.n_chunks, w.layout), "block", mask=mask2,
                                order="lpt_device", stream=side)
    o2 = G.empty_like_qkv(q)
    with torch.cuda.stream(side):
        bd.sparse_attn_fwd(plan2, q, k, v, 0, w.n_chunks, o=o2)
    torch.cuda.synchronize()
    rows = G.sample_rows(w, 64, seed=9)
    idx = tuple(np.array(rows).T)
    ref1, _ = A.masked_attention(w.q, w.k, w.v, w.mask, w.block, rows=rows)
    ref2, _ = A.masked_attention(w.q, w.k, w.v, w2.mask, w.block, rows=rows)
    G.assert_close(G.to64(o1)[idx], ref1, G.BF16_TOL, "plan 1 (destroyed while running)")
    G.assert_close(G.to64(o2)[idx], ref2, G.BF16_TOL, "plan 2 (reused buffers)")
    plan2.close()
