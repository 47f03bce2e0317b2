"""GPU parity of the device planner (SA_ORDER_LPT_DEVICE: round-based LPT made on the GPU
with no host round trip) against the oracle's lpt_rounds, through the C ABI.  Lists, bin
pointers and bin loads are compared bit-exactly for the full range and every chunk; the
attention outputs under a device plan must equal those under the host plan bit for bit
(an item's output does not depend on which workgroup runs it or when)."""
import numpy as np
import pytest
import torch

from oracle import plan as P
from sparse_mask_load_amd import binding as bd
from sparse_mask_load_amd import workloads as W
from tests import gpu_util as G

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    bd.lib()


def _check_device_lists(w, plan, layout=None):
    layout = layout or w.layout
    info = bd.sparse_attn_plan_info(plan)
    m, n, C = info["num_bins"], w.B * w.H * w.nQ, w.n_chunks
    ref = P.popcount(w.mask, C, layout)
    assert info["total_live"] == info["load_sum"] == ref["total"]
    lists = [(-1, ref["row"])] + [(c, ref["crow"][:, :, c, :]) for c in range(C)]
    for chunk, loads in lists:
        want = P.plan_items(loads, m, "lpt_device")
        items = bd.sparse_attn_plan_copy(plan, bd.SA_PLAN_ITEMS, n, chunk)
        ptr = bd.sparse_attn_plan_copy(plan, bd.SA_PLAN_BIN_PTR, m + 1, chunk)
        bl = bd.sparse_attn_plan_copy(plan, bd.SA_PLAN_BIN_LOAD, m, chunk)
        assert np.array_equal(ptr, want["bin_ptr"]), f"bin_ptr of list {chunk}"
        assert np.array_equal(items, want["items"]), f"items of list {chunk}"
        assert np.array_equal(bl, want["bin_load"]), f"bin loads of list {chunk}"
    row = ref["row"].reshape(-1)
    assert info["makespan"] == P.plan_items(ref["row"], m, "lpt_device")["makespan"]
    assert info["lower_bound"] == max(int(row.max()), -(-int(row.sum()) // m))
    return info


@pytest.mark.parametrize("wid", [1, 2, 3, 4])
def test_device_plan_lists_and_outputs_match(wid):
    w = W.make(wid)
    q, k, v = G.upload(w)
    bins = 2 if wid == 1 else 0
    pd = G.plan_block(w, q, order="lpt_device", num_bins=bins)
    info = _check_device_lists(w, pd)
    if wid in (3, 4):  # the round rule reaches the LPT makespan on these masks
        ph = G.plan_block(w, q, order="lpt", num_bins=bins)
        assert info["makespan"] == bd.sparse_attn_plan_info(ph)["makespan"] == info["lower_bound"]
    else:
        ph = G.plan_block(w, q, order="lpt", num_bins=bins)
    o_d = G.run_full(pd, q, k, v)
    o_h = G.run_full(ph, q, k, v)
    assert torch.equal(o_d, o_h)
    op_d, mp_d, lp_d = G.run_partial(pd, q, k, v, 0, w.n_chunks)
    op_h, mp_h, lp_h = G.run_partial(ph, q, k, v, 0, w.n_chunks)
    assert torch.equal(mp_d, mp_h) and torch.equal(lp_d, lp_h) and torch.equal(op_d, op_h)
    del op_d, op_h
    # one ring step at a time uses the chunk's own device list
    c = w.n_chunks - 1
    o1, m1, l1 = G.run_partial(pd, q, k, v, c, c + 1)
    assert torch.equal(m1[0], mp_d[c]) and torch.equal(l1[0], lp_d[c])


@pytest.mark.parametrize("bins", [1, 3, 7, 64, 100, 1000, 1024])
def test_device_plan_bin_counts(bins):
    """Bin counts around the shuffle / LDS-exchange boundary of the in-register sort
    (64), non-powers of two, and the limit."""
    w = W.make_custom(2, 3, 1000, 64, block=64, n_chunks=2, pattern="zipf", density=0.4, seed=bins)
    q, k, v = G.upload(w)
    pd = G.plan_block(w, q, order="lpt_device", num_bins=bins)
    _check_device_lists(w, pd)
    ph = G.plan_block(w, q, order="lpt", num_bins=bins)
    assert torch.equal(G.run_full(pd, q, k, v), G.run_full(ph, q, k, v))


def test_device_plan_striped_and_token_causal():
    w = W.make_custom(1, 4, 2048, 128, block=128, n_chunks=4, pattern="causal", layout="striped", seed=5)
    q, k, v = G.upload(w)
    pd = G.plan_block(w, q, order="lpt_device", token_causal=True)
    _check_device_lists(w, pd)
    ph = G.plan_block(w, q, order="lpt", token_causal=True)
    assert torch.equal(G.run_full(pd, q, k, v), G.run_full(ph, q, k, v))


def test_device_plan_largest_list():
    """16384 items (the limit): 64 heads of 256 Q-blocks."""
    w = W.make_custom(1, 64, 32768, 128, block=128, n_chunks=1, pattern="zipf", density=0.3, seed=11,
                      mask_only=True)
    q = torch.empty((1, 64, 32768, 128), dtype=torch.bfloat16, device="cuda")
    pd = G.plan_block(w, q, order="lpt_device")
    _check_device_lists(w, pd)


def test_device_plan_limits():
    w = W.make_custom(1, 65, 16384, 64, block=64, n_chunks=1, pattern="ones", seed=1, mask_only=True)  # 16640 items
    q = torch.empty((1, 65, 16384, 64), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(bd.SparseAttnError) as e:
        G.plan_block(w, q, order="lpt_device")
    assert e.value.status == bd.SA_ERR_UNSUPPORTED
    w2 = W.make_custom(1, 1, 256, 64, block=64, pattern="ones", seed=1)
    q2, _, _ = G.upload(w2)
    with pytest.raises(bd.SparseAttnError) as e:
        G.plan_block(w2, q2, order="lpt_device", num_bins=1025)
    assert e.value.status == bd.SA_ERR_UNSUPPORTED


def test_device_plan_on_side_stream_without_host_wait():
    w = W.make(3)
    q, k, v = G.upload(w)
    mask = torch.from_numpy(np.ascontiguousarray(w.mask)).cuda()
    prob = bd.make_problem(q, w.block, w.n_chunks, w.layout)
    ref = G.run_full(G.plan_block(w, q), q, k, v)
    side = torch.cuda.Stream()
    o = G.empty_like_qkv(q)
    plans = []
    for _ in range(3):  # plans made on the side stream, each forward on the main stream waits on its plan
        p = bd.sparse_attn_plan(prob, "block", mask=mask, order="lpt_device", stream=side)
        bd.sparse_attn_fwd(p, q, k, v, 0, w.n_chunks, o=o)
        plans.append(p)
    torch.cuda.synchronize()
    assert torch.equal(o, ref)
    for p in plans:
        p.close()
