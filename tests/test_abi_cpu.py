"""CPU checks of the C ABI: the library loads, exports every declared entry point, its host
LPT planner is bit-exact against the oracle, and argument errors are reported before any
GPU work.  No kernel is launched here."""
import ctypes
import os
import re

import numpy as np
import pytest

from oracle import plan as P
from sparse_mask_load_amd import binding as bd
from sparse_mask_load_amd import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    text = open(os.path.join(ROOT, "include", "sparse_attn.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:sa_status|void|const char\s*\*)\s+(\w+)\s*\(", text, flags=re.M)))


def test_library_exports_every_declared_symbol():
    names = _declared_functions()
    assert {"sparse_attn_plan", "sparse_attn_fwd", "chunk_merge"} <= set(names)
    lib = bd.lib()
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(bd._SIGNATURES)


def test_status_strings():
    assert bd.sa_status_string(0) == "SA_OK"
    for st in (-1, -2, -3, -4):
        assert bd.sa_status_string(st).startswith("SA_ERR")


def _oracle_lists(loads, m, order):
    bins, bl = (P.lpt if order == "lpt" else P.naive)(list(loads), m)
    items = [j for b in bins for j in b]
    ptr = np.cumsum([0] + [len(b) for b in bins])
    return np.array(items), ptr, np.array(bl)


@pytest.mark.parametrize("order", ["lpt", "naive"])
def test_host_assign_bit_exact_random(order):
    rng = np.random.default_rng(0)
    for trial in range(40):
        n = int(rng.integers(0, 400))
        m = int(rng.integers(1, 40))
        loads = rng.integers(0, int(rng.integers(1, 60)), size=n)
        items, ptr, bl = bd.sparse_attn_assign_host(loads, m, order)
        oi, op, ob = _oracle_lists(loads, m, order)
        assert np.array_equal(items, oi) and np.array_equal(ptr, op) and np.array_equal(bl, ob)


def test_host_assign_bit_exact_large_loads():
    """Loads beyond the counting-sort and load-bucket ranges take the comparison-sort and heap paths."""
    rng = np.random.default_rng(1)
    for trial in range(10):
        n = int(rng.integers(1, 300))
        m = int(rng.integers(1, 33))
        loads = rng.integers(0, 10 ** 9, size=n)
        loads[: n // 3] = rng.integers(0, 3, size=n // 3)  # with many small and equal loads
        items, ptr, bl = bd.sparse_attn_assign_host(loads, m, "lpt")
        oi, op, ob = _oracle_lists(loads, m, "lpt")
        assert np.array_equal(items, oi) and np.array_equal(ptr, op) and np.array_equal(bl, ob)


def test_host_assign_page_example():
    items, ptr, bl = bd.sparse_attn_assign_host([8, 7, 6, 5, 4], 2)
    assert items.tolist() == [0, 3, 4, 1, 2] and ptr.tolist() == [0, 3, 5] and bl.tolist() == [17, 13]


@pytest.mark.parametrize("cfg,m", [(2, 512), (3, 256), (4, 256)])
def test_host_assign_bit_exact_on_workload_rows(cfg, m):
    w = W.make(cfg, with_data=False)
    cnt = P.popcount(w.mask, w.n_chunks)
    for order in ("lpt", "naive"):
        loads = cnt["row"].reshape(-1)
        items, ptr, bl = bd.sparse_attn_assign_host(loads, m, order)
        ref = P.plan_items(cnt["row"], m, order)
        assert np.array_equal(items, ref["items"]) and np.array_equal(ptr, ref["bin_ptr"])
        assert np.array_equal(bl, ref["bin_load"])
    if cfg == 3:
        # causal block mask over 256 workgroups: LPT reaches the lower bound exactly
        ref = P.plan_items(cnt["row"], 256, "lpt")
        assert ref["makespan"] == 516 == -(-cnt["total"] // 256)
        naive = P.plan_items(cnt["row"], 256, "naive")
        assert naive["makespan"] / (cnt["total"] / 256) > 1.9


def test_host_assign_errors():
    with pytest.raises(bd.SparseAttnError) as e:
        bd.sparse_attn_assign_host([1, 2], 0)
    assert e.value.status == bd.SA_ERR_INVALID
    with pytest.raises(bd.SparseAttnError) as e:
        bd.sparse_attn_assign_host([1, -2], 3)
    assert e.value.status == bd.SA_ERR_INVALID and "loads[1]" in str(e.value)


def _problem(**kw):
    base = dict(B=1, H=2, S=256, D=64, block=64, n_chunks=2, layout=0, dtype=bd.SA_BF16, scale=0.0, token_causal=0,
                sb=2 * 256 * 64, sh=256 * 64, ss=64)
    base.update(kw)
    return bd.sa_problem(**base)


BAD_PROBLEMS = [
    (dict(D=96), bd.SA_ERR_UNSUPPORTED),
    (dict(block=32), bd.SA_ERR_UNSUPPORTED),
    (dict(B=0), bd.SA_ERR_INVALID),
    (dict(n_chunks=3), bd.SA_ERR_INVALID),
    (dict(n_chunks=0), bd.SA_ERR_INVALID),
    (dict(ss=32), bd.SA_ERR_INVALID),
    (dict(layout=1, n_chunks=4), bd.SA_ERR_UNSUPPORTED),  # block/C = 16 keys < 32
    (dict(layout=7), bd.SA_ERR_INVALID),
    (dict(dtype=bd.SA_F32, block=128), bd.SA_ERR_UNSUPPORTED),
    # Q-block pairs: bf16, block 128, contiguous layout, S a multiple of 128
    (dict(q_pairs=1), bd.SA_ERR_UNSUPPORTED),  # block 64
    (dict(q_pairs=1, block=128, S=320, n_chunks=1, sb=2 * 320 * 64, sh=320 * 64), bd.SA_ERR_UNSUPPORTED),
    (dict(q_pairs=1, block=64, dtype=bd.SA_F32), bd.SA_ERR_UNSUPPORTED),
]


@pytest.mark.parametrize("kw,status", BAD_PROBLEMS)
def test_plan_rejects_bad_problems_before_touching_the_gpu(kw, status):
    import ctypes
    prob = _problem(**kw)
    sp = bd.sa_sparsity(bd.SA_KIND_BLOCK, 0, 0, 0, 1, None, None, None, None, None, None)
    out = ctypes.c_void_p()
    st = bd.lib().sparse_attn_plan(ctypes.byref(prob), ctypes.byref(sp), 0, 0, ctypes.byref(out), None)
    assert st == status, bd.sa_last_error()
    assert out.value is None


def _plan_status(prob, kind=bd.SA_KIND_BLOCK, order=0, num_bins=0):
    import ctypes
    sp = bd.sa_sparsity(kind, 32, 8, 1, 1, 1, 1, 1, 1, None, None)
    out = ctypes.c_void_p()
    st = bd.lib().sparse_attn_plan(ctypes.byref(prob), ctypes.byref(sp), num_bins, order, ctypes.byref(out), None)
    assert out.value is None
    return st


def test_problem_fields_are_the_declared_ones():
    # a misspelt keyword would become a plain Python attribute and leave the field at 0
    names = [n for n, _ in bd.sa_problem._fields_]
    assert names == ["B", "H", "S", "D", "block", "n_chunks", "layout", "dtype", "scale", "token_causal",
                     "q_pairs", "sb", "sh", "ss"]
    # q_pairs takes the padding after token_causal: the C struct keeps its size and offsets
    assert ctypes.sizeof(bd.sa_problem) == 72 and bd.sa_problem.sb.offset == 48


def test_token_causal_only_for_block_plans():
    assert _plan_status(_problem(token_causal=1), kind=bd.SA_KIND_TOPK) == bd.SA_ERR_INVALID
    assert "token_causal" in bd.sa_last_error()


def test_hip_errors_surface_as_sa_err_hip():
    """A HIP runtime failure comes back as SA_ERR_HIP with the runtime's text (here: no device
    on this machine), from the plan call and from a launch."""
    import torch
    if torch.cuda.device_count() > 0:
        pytest.skip("a device is visible; this failure path needs a machine without one")
    mask = np.ones((1, 2, 4, 4), np.uint8)
    sp = bd.sa_sparsity(bd.SA_KIND_BLOCK, 0, 0, 0, mask.ctypes.data, None, None, None, None, None, None)
    out = ctypes.c_void_p()
    st = bd.lib().sparse_attn_plan(ctypes.byref(_problem()), ctypes.byref(sp), 0, 0, ctypes.byref(out), None)
    assert st == bd.SA_ERR_HIP and out.value is None
    assert "hip" in bd.sa_last_error().lower()
    arr = (bd._P * 1)(1)
    assert bd.lib().chunk_merge(1, arr, arr, arr, 10, 64, None, 1, None, None) == bd.SA_ERR_INVALID  # NULL output
    assert bd.lib().chunk_merge(1, arr, arr, arr, 10, 64, 1, 1, None, None) == bd.SA_ERR_HIP
    assert "launch_merge" in bd.sa_last_error()  # the failing call, then the runtime's text


def test_q_pairs_only_for_block_plans():
    assert _plan_status(_problem(q_pairs=1), kind=bd.SA_KIND_TOPK) == bd.SA_ERR_INVALID
    assert "q_pairs" in bd.sa_last_error()


@pytest.mark.parametrize("order", [bd.SA_ORDER_LPT_DEVICE, bd.SA_ORDER_LPT_DYNAMIC], ids=["device", "dynamic"])
def test_device_order_limits_checked_before_the_gpu(order):
    # 65 heads of 256 Q-blocks = 16640 items, above the device planner's 16384
    big = _problem(H=65, S=16384, sb=65 * 16384 * 64, sh=16384 * 64, n_chunks=1)
    assert _plan_status(big, order=order) == bd.SA_ERR_UNSUPPORTED
    assert "16384" in bd.sa_last_error()
    assert _plan_status(_problem(), order=order, num_bins=1025) == bd.SA_ERR_UNSUPPORTED
    # with Q-block pairs the limit counts pairs: 129 heads of 128 pairs = 16512 items
    pairs = _problem(H=129, S=32768, block=128, q_pairs=1, sb=129 * 32768 * 64, sh=32768 * 64, n_chunks=1)
    assert _plan_status(pairs, order=order) == bd.SA_ERR_UNSUPPORTED
    assert "16384" in bd.sa_last_error()
    assert _plan_status(_problem(), order=5) == bd.SA_ERR_INVALID
    # the run-time queue exists only for block plans
    assert _plan_status(_problem(), kind=bd.SA_KIND_TOPK, order=bd.SA_ORDER_LPT_DYNAMIC) == bd.SA_ERR_INVALID
    assert "block plans" in bd.sa_last_error()


def test_fwd_and_merge_argument_errors():
    lib = bd.lib()
    assert lib.sparse_attn_fwd(None, 1, 1, 1, 0, 1, 1, None, None, None, None, None) == bd.SA_ERR_INVALID
    assert "plan is NULL" in bd.sa_last_error()
    arr = (bd._P * 1)(1)
    assert lib.chunk_merge(0, arr, arr, arr, 10, 64, 1, 0, None, None) == bd.SA_ERR_INVALID
    assert lib.chunk_merge(1, arr, arr, arr, 10, 96, 1, 0, None, None) == bd.SA_ERR_UNSUPPORTED
    assert lib.chunk_merge(1, arr, arr, arr, 0, 64, 1, 0, None, None) == bd.SA_OK  # nothing to do
    lib.sparse_attn_plan_destroy(None)  # no-op


def test_host_grouped_assign_bit_exact_random():
    """Two-level (XCD-affine) LPT: the library's host code equals the oracle's definition."""
    rng = np.random.default_rng(3)
    for trial in range(40):
        heads = int(rng.integers(0, 12))
        per = int(rng.integers(1, 30))
        groups = int(rng.choice([1, 2, 4, 8]))
        m = groups * int(rng.integers(1, 6)) + (int(rng.integers(0, 2)) if trial % 5 == 0 else 0)
        loads = rng.integers(0, int(rng.integers(1, 50)), size=heads * per)
        items, ptr, bl = bd.sparse_attn_assign_host_grouped(loads, per, m, groups)
        bins, ref_bl = P.lpt_grouped(loads.tolist(), per, m, groups)
        assert np.array_equal(items, [j for b in bins for j in b])
        assert np.array_equal(ptr, np.cumsum([0] + [len(b) for b in bins]))
        assert np.array_equal(bl, ref_bl)


@pytest.mark.parametrize("cfg,m", [(3, 256), (4, 256)])
def test_host_grouped_assign_on_workload_rows(cfg, m):
    w = W.make(cfg, with_data=False)
    cnt = P.popcount(w.mask, w.n_chunks)
    items, ptr, bl = bd.sparse_attn_assign_host_grouped(cnt["row"], w.nQ, m, 8)
    ref = P.plan_items(cnt["row"], m, "lpt_xcd", groups=8)
    assert np.array_equal(items, ref["items"]) and np.array_equal(ptr, ref["bin_ptr"])
    assert np.array_equal(bl, ref["bin_load"])
    # every head's items land in one group of bins (b mod 8)
    heads = cnt["row"].reshape(-1, w.nQ).shape[0]
    bin_of = np.empty(heads * w.nQ, np.int64)
    for b in range(m):
        bin_of[items[ptr[b]:ptr[b + 1]]] = b
    assert all(len(set((bin_of[h * w.nQ:(h + 1) * w.nQ] % 8).tolist())) == 1 for h in range(heads))


def test_noalloc_argument_errors_before_the_gpu():
    """The allocation-free entry point rejects bad arguments and sizes beyond its work array
    before any HIP call."""
    lib = bd.lib()
    mask = np.ones(4096, np.uint8)
    ptr = mask.ctypes.data + (-mask.ctypes.data) % 16  # 16-byte aligned host address (never dereferenced)
    call = lambda prob, m=ptr, bins=0, c0=0, c1=1, o=1: lib.sparse_attn_fwd_noalloc(
        ctypes.byref(prob), m, bins, 1, 1, 1, c0, c1, o, None, None, None, None)
    ok = _problem()
    assert call(ok, m=None) == bd.SA_ERR_INVALID
    assert call(ok, m=ptr + 1) == bd.SA_ERR_INVALID and "aligned" in bd.sa_last_error()
    assert call(ok, c0=1, c1=1) == bd.SA_ERR_INVALID
    assert call(ok, o=None) == bd.SA_ERR_INVALID and "partial mode" in bd.sa_last_error()
    assert call(ok, bins=-1) == bd.SA_ERR_INVALID
    assert call(ok, bins=1025) == bd.SA_ERR_UNSUPPORTED
    big = _problem(H=65, S=16384, sb=65 * 16384 * 64, sh=16384 * 64, n_chunks=1)
    assert call(big) == bd.SA_ERR_UNSUPPORTED and "16384" in bd.sa_last_error()
    # 64 heads x 256 Q-blocks x 64 chunks of counts do not fit the 2 MiB work array
    wide = _problem(H=64, S=16384, sb=64 * 16384 * 64, sh=16384 * 64, n_chunks=64)
    assert call(wide) == bd.SA_ERR_UNSUPPORTED and "work array" in bd.sa_last_error()
