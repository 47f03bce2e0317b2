"""GPU parity of the run-time LPT queue (SA_ORDER_LPT_DYNAMIC).

The plan's queue of every list (the full range and each chunk) must equal the oracle's LPT
order of that list's loads (``oracle/plan.py: lpt_order``, the LPT paragraph's greedy in its
list-scheduling form), and its bin lists those of the device planner.  Forward calls that take
the queue must give the same output bits as the device planner's static lists: an item is
computed the same way whichever workgroup takes it.  Launches are repeated, since each one's
last workgroup returns the queue's counters to zero for the next.
"""
import threading

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
    bd.lib()  # fails loudly if the library is missing


def _check_queues(w, plan, q_pairs):
    info = bd.sparse_attn_plan_info(plan)
    B, H, C, n = w.B, w.H, w.n_chunks, info["n_items"]
    nI = (info["nQ"] + 1) // 2 if q_pairs else info["nQ"]
    row = bd.sparse_attn_plan_copy(plan, bd.SA_PLAN_PAIR_ROW if q_pairs else bd.SA_PLAN_ROW, B * H * nI)
    crow = bd.sparse_attn_plan_copy(plan, bd.SA_PLAN_PAIR_CROW if q_pairs else bd.SA_PLAN_CROW,
                                    B * H * C * nI).reshape(B * H, C, nI)
    lists = [(-1, row)] + [(c, crow[:, c, :].reshape(-1)) for c in range(C)]
    for chunk, loads in lists:
        queue = bd.sparse_attn_plan_copy(plan, bd.SA_PLAN_LPT_ORDER, n, chunk)
        want = P.plan_items(loads.reshape(B * H, nI), info["num_bins"], "lpt_dynamic")
        assert np.array_equal(queue, want["queue"]), f"queue of list {chunk}"
        items = bd.sparse_attn_plan_copy(plan, bd.SA_PLAN_ITEMS, n, chunk)
        ptr = bd.sparse_attn_plan_copy(plan, bd.SA_PLAN_BIN_PTR, info["num_bins"] + 1, chunk)
        assert np.array_equal(items, want["items"]) and np.array_equal(ptr, want["bin_ptr"])


def _same_outputs(w, q, k, v, plan_s, plan_d, reps=3):
    C = w.n_chunks
    o_ref = G.run_full(plan_s, q, k, v)
    part_ref = G.run_partial(plan_s, q, k, v, 0, C)
    one_ref = [G.run_partial(plan_s, q, k, v, c, c + 1) for c in range(C)]
    for rep in range(reps):
        assert torch.equal(G.run_full(plan_d, q, k, v), o_ref), f"full mode, launch {rep}"
        for got, ref in zip(G.run_partial(plan_d, q, k, v, 0, C), part_ref):
            assert torch.equal(got, ref), f"partial mode, launch {rep}"
        for c in range(C):
            for got, ref in zip(G.run_partial(plan_d, q, k, v, c, c + 1), one_ref[c]):
                assert torch.equal(got, ref), f"chunk {c} alone, launch {rep}"


DYN_CASES = [
    # (B, H, S, D, block, C, pattern, density, q_pairs, token_causal, layout)
    (1, 3, 1024, 128, 128, 4, "causal", 0.0, True, False, "contiguous"),      # pair kernel
    (1, 3, 1152, 128, 128, 3, "bernoulli", 0.5, False, False, "contiguous"),  # single items
    (2, 2, 1024, 128, 128, 4, "zipf", 0.4, False, True, "contiguous"),        # single items, token-causal
    (1, 2, 2048, 128, 128, 4, "causal", 0.0, True, False, "striped"),         # striped pairs
    (1, 2, 1024, 64, 64, 2, "bernoulli", 0.4, False, False, "contiguous"),    # block 64: bin lists
    (1, 2, 1000, 128, 128, 2, "causal", 0.0, False, False, "contiguous"),     # ragged S: bin lists
]


@pytest.mark.parametrize("n", range(len(DYN_CASES)),
                         ids=[f"{c[6]}-S{c[2]}-b{c[4]}-C{c[5]}-{'pairs' if c[8] else 'single'}"
                              f"{'-tc' if c[9] else ''}-{c[10][:4]}" for c in DYN_CASES])
def test_dynamic_queue_small(n):
    B, H, S, D, blk, C, pattern, dens, qp, tc, layout = DYN_CASES[n]
    print(f"dynamic case {n}: {DYN_CASES[n]}", flush=True)
    w = W.make_custom(B, H, S, D, block=blk, n_chunks=C, dtype="bf16", pattern=pattern, density=dens,
                      seed=700 + n, layout=layout)
    q, k, v = G.upload(w)
    plan_s = G.plan_block(w, q, order="lpt_device", token_causal=tc, q_pairs=qp)
    plan_d = G.plan_block(w, q, order="lpt_dynamic", token_causal=tc, q_pairs=qp)
    _check_queues(w, plan_d, qp)
    _same_outputs(w, q, k, v, plan_s, plan_d)
    # fewer workgroups than items: every workgroup takes several
    plan_d7 = G.plan_block(w, q, order="lpt_dynamic", num_bins=7, token_causal=tc, q_pairs=qp)
    _same_outputs(w, q, k, v, plan_s, plan_d7, reps=2)
    for p in (plan_s, plan_d, plan_d7):
        p.close()


@pytest.mark.parametrize("q_pairs", [True, False], ids=["pairs", "single"])
def test_dynamic_queue_causal_workload(q_pairs):
    """The causal workload (1024 pair items or 2048 single items over 256 workgroups): the queue
    against the oracle and the outputs against the device planner's lists, bit for bit."""
    w = W.make(3)
    q, k, v = G.upload(w)
    plan_s = G.plan_block(w, q, order="lpt_device", q_pairs=q_pairs)
    plan_d = G.plan_block(w, q, order="lpt_dynamic", q_pairs=q_pairs)
    _check_queues(w, plan_d, q_pairs)
    o_ref = G.run_full(plan_s, q, k, v)
    part_ref = G.run_partial(plan_s, q, k, v, 0, w.n_chunks)
    for rep in range(3):
        assert torch.equal(G.run_full(plan_d, q, k, v), o_ref), f"full mode, launch {rep}"
        for got, ref in zip(G.run_partial(plan_d, q, k, v, 0, w.n_chunks), part_ref):
            assert torch.equal(got, ref), f"partial mode, launch {rep}"
    plan_s.close()
    plan_d.close()


def test_dynamic_queue_two_host_threads():
    """Forward calls on one run-time-order plan from two host threads, each on a stream of its
    own, share the queue's counters, so the library runs them one after another: every output
    equals the static order's bit for bit."""
    w = W.make_custom(1, 4, 2048, 128, block=128, n_chunks=4, dtype="bf16", pattern="causal", density=0.0,
                      seed=790)
    q, k, v = G.upload(w)
    plan_s = G.plan_block(w, q, order="lpt_device", q_pairs=True)
    plan_d = G.plan_block(w, q, order="lpt_dynamic", q_pairs=True)
    o_ref = G.run_full(plan_s, q, k, v)
    streams = [torch.cuda.Stream() for _ in range(2)]
    outs = [[G.empty_like_qkv(q) for _ in range(8)] for _ in range(2)]
    torch.cuda.synchronize()
    errors = []

    def worker(i):
        try:
            for o in outs[i]:
                bd.sparse_attn_fwd(plan_d, q, k, v, o=o, stream=streams[i])
        except Exception as e:  # reported by the main thread
            errors.append(e)

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(2)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    torch.cuda.synchronize()
    assert not errors, errors
    for i in range(2):
        for j, o in enumerate(outs[i]):
            assert torch.equal(o, o_ref), f"thread {i}, call {j}"
    plan_s.close()
    plan_d.close()
