"""Pins of oracle.plan: popcounts, LPT, naive order, brute force, ring step table."""
import itertools
import random

import numpy as np
import pytest

from oracle import plan as P
from sparse_mask_load_amd import workloads as W


def _parse_partition(text):
    return [sorted((int(x) for x in part.split()), reverse=True) for part in text.split("|")]


def test_lpt_counter_example_from_page(golden):
    g = golden("lpt_counter_example.txt")
    loads = [int(x) for x in g["loads"].split()]
    m = int(g["machines"])
    bins, bin_load = P.lpt(loads, m)
    got = [sorted((loads[j] for j in b), reverse=True) for b in bins]
    assert got == _parse_partition(g["lpt_partition"])
    assert max(bin_load) == int(g["lpt_makespan"])
    opt, assign = P.brute_force_makespan(loads, m)
    assert opt == int(g["opt_makespan"])
    parts = [sorted((loads[j] for j in range(len(loads)) if assign[j] == b), reverse=True)
             for b in range(m)]
    assert sorted(parts) == sorted(_parse_partition(g["opt_partition"]))


def test_lpt_within_worst_case_bound(golden):
    g = golden("lpt_bound.txt")
    assert g["bound_numerator"] == "4m-1" and g["bound_denominator"] == "3m"
    rng = random.Random(1234)
    worst = {}
    for trial in range(400):
        m = rng.randint(2, 3)
        n = rng.randint(1, 8 if m == 2 else 7)
        loads = [rng.randint(0, 12) for _ in range(n)]
        _, bl = P.lpt(loads, m)
        opt, _ = P.brute_force_makespan(loads, m)
        if opt == 0:
            assert max(bl) == 0
            continue
        ratio = max(bl) / opt
        assert ratio <= (4 * m - 1) / (3 * m) + 1e-12, (loads, m)
        worst[m] = max(worst.get(m, 1.0), ratio)
    assert worst[2] >= 1.0


@pytest.mark.parametrize("m,loads,lpt_span,opt_span", [
    # Graham's tight instances for the LPT bound (textbook, Graham 1969): 2m+1 jobs.
    (2, [3, 3, 2, 2, 2], 7, 6),
    (3, [5, 5, 4, 4, 3, 3, 3], 11, 9),
])
def test_lpt_reaches_bound_on_tight_instances(m, loads, lpt_span, opt_span):
    _, bl = P.lpt(loads, m)
    opt, _ = P.brute_force_makespan(loads, m)
    assert max(bl) == lpt_span and opt == opt_span
    assert max(bl) * 3 * m == opt * (4 * m - 1)


def test_lpt_tie_rules():
    # equal loads: item ids ascending go to bins 0, 1, 2, ...; then back to the lowest bin
    bins, bl = P.lpt([5, 5, 5, 5, 5], 3)
    assert bins == [[0, 3], [1, 4], [2]] and bl == [10, 10, 5]
    # zero loads are still placed (they go to the least-loaded bins)
    bins, bl = P.lpt([0, 4, 0], 2)
    assert bins == [[1], [0, 2]] and bl == [4, 0]


def test_lpt_is_list_scheduling_of_sorted_jobs():
    # Invariant: every job lands on a bin whose load, just before it, was minimal.
    rng = np.random.default_rng(7)
    loads = rng.integers(0, 50, size=300).tolist()
    m = 17
    bins, bl = P.lpt(loads, m)
    where = {j: b for b, lst in enumerate(bins) for j in lst}
    order = sorted(range(len(loads)), key=lambda i: (-loads[i], i))
    cur = [0] * m
    for j in order:
        b = where[j]
        assert cur[b] == min(cur)
        assert b == cur.index(min(cur))
        cur[b] += loads[j]
    assert cur == bl
    assert sorted(j for lst in bins for j in lst) == list(range(len(loads)))


def test_lpt_order_and_list_scheduling():
    # the queue of the run-time order: loads descending, ids ascending on ties (hand example)
    assert P.lpt_order([3, 7, 3, 0, 7]) == [1, 4, 0, 2, 3]
    # list scheduling of that queue with run times equal to the loads is the LPT greedy
    rng = np.random.default_rng(11)
    for m in (1, 2, 5, 17):
        loads = rng.integers(0, 60, size=200).tolist()
        assert P.list_schedule(P.lpt_order(loads), loads, m) == P.lpt(loads, m)[0]
    # page example: [8,7,6,5,4] on two machines -> 8+5+4 | 7+6
    assert P.list_schedule(P.lpt_order([8, 7, 6, 5, 4]), [8, 7, 6, 5, 4], 2) == [[0, 3, 4], [1, 2]]
    # with other run times a machine that finishes early takes more of the queue
    times = [10, 10, 1, 1, 1, 1]
    assert P.list_schedule([0, 1, 2, 3, 4, 5], [20, 10, 1, 1, 1, 1], 2) == [[0], [1, 2, 3, 4, 5]]
    assert P.list_schedule([0, 1, 2, 3, 4, 5], times, 2) == [[0, 2, 4], [1, 3, 5]]
    q = P.plan_items(np.array([[3, 7, 3, 0, 7]]), 2, "lpt_dynamic")
    assert q["queue"].tolist() == [1, 4, 0, 2, 3]
    assert np.array_equal(q["items"], P.plan_items(np.array([[3, 7, 3, 0, 7]]), 2, "lpt_device")["items"])


def test_naive_round_robin():
    bins, bl = P.naive([1, 2, 3, 4, 5, 6, 7], 3)
    assert bins == [[0, 3, 6], [1, 4], [2, 5]] and bl == [12, 7, 9]


def _brute_counts(mask, n_chunks, layout):
    B, H, nQ, nK = mask.shape
    row = np.zeros((B, H, nQ), int)
    col = np.zeros((B, H, nK), int)
    crow = np.zeros((B, H, n_chunks, nQ), int)
    for b in range(B):
        for h in range(H):
            for i in range(nQ):
                for j in range(nK):
                    if mask[b, h, i, j]:
                        row[b, h, i] += 1
                        col[b, h, j] += 1
                        if layout == "contiguous":
                            crow[b, h, j // (nK // n_chunks), i] += 1
                        else:
                            for c in range(n_chunks):
                                crow[b, h, c, i] += 1
    return row, col, crow


@pytest.mark.parametrize("layout", ["contiguous", "striped"])
def test_popcount_brute_force(layout):
    rng = np.random.default_rng(3)
    mask = (rng.random((2, 3, 8, 8)) < 0.4).astype(np.uint8) * rng.integers(1, 255, (2, 3, 8, 8)).astype(np.uint8)
    cnt = P.popcount(mask, 4, layout)
    row, col, crow = _brute_counts(mask, 4, layout)
    assert (cnt["row"] == row).all() and (cnt["col"] == col).all() and (cnt["crow"] == crow).all()
    assert cnt["total"] == row.sum() == col.sum()


def test_popcount_row_and_column_sums_4x4():
    # db-SP scenario 2 uses a 4x4 mask: Q-block load = row sum, KV-block load = column sum
    # (values below counted by hand).
    mask = np.array([[[[1, 0, 0, 0], [1, 1, 0, 0], [0, 1, 1, 0], [1, 1, 1, 1]]]], np.uint8)
    cnt = P.popcount(mask, 2)
    assert cnt["row"][0, 0].tolist() == [1, 2, 2, 4]
    assert cnt["col"][0, 0].tolist() == [3, 3, 2, 1]
    assert cnt["crow"][0, 0].tolist() == [[1, 2, 1, 2], [0, 0, 1, 2]]


def test_workload_tile_counts():
    w2 = W.make(2, with_data=False)
    cnt = P.popcount(w2.mask, 4)
    # frame band: 4 rows per frame x (14 frames x 12 live blocks + 2 edge frames x 8) = 736
    assert (cnt["row"][0, :12].sum(axis=1) == 736).all()
    assert (np.diagonal(w2.mask[0, 12:], axis1=1, axis2=2) == 1).all()
    w3 = W.make(3, with_data=False)
    cnt3 = P.popcount(w3.mask, 4)
    assert (cnt3["row"].sum(axis=2) == 128 * 129 // 2).all() and cnt3["total"] == 132096
    # per-chunk work of contiguous causal chunks: 3600 / 2576 / 1552 / 528 tiles per head
    assert cnt3["crow"][0, 0].sum(axis=1).tolist() == [3600, 2576, 1552, 528]


def test_ring_step_table_matches_page(golden):
    g = golden("causal_ring_steps.txt")
    cp = int(g["cp"])
    w3 = W.make(3, with_data=False)
    tab = P.step_table(w3.mask[:, :1], w3.S, w3.block, cp, "contiguous")[0, 0]
    nonzero = tab > 0
    assert nonzero.size == int(g["steps_total"])
    assert int(nonzero.sum()) == int(g["steps_with_work"])
    assert nonzero.sum(axis=1).tolist() == [int(x) for x in g["steps_per_gpu"].split()]
    assert 100.0 * nonzero.sum() / nonzero.size == float(g["fraction_percent"])
    assert 100.0 - 100.0 * nonzero.sum() / nonzero.size == float(g["saved_percent"])
    # striped: every step has work and the causal work is balanced
    tab_s = P.step_table(w3.mask[:, :1], w3.S, w3.block, cp, "striped")[0, 0]
    assert (tab_s > 0).all()
    assert len(set(tab_s.ravel().tolist())) == 1
    assert tab_s.sum() == tab.sum() == 8256 * 128 * 128
    # imbalance of the contiguous per-GPU work vs the striped one
    assert tab.sum(axis=1).max() > tab.sum(axis=1).min() * 2
    assert tab_s.sum(axis=1).max() == tab_s.sum(axis=1).min()


def test_plan_items_ids_and_ptrs():
    row = np.array([[[3, 1, 2], [0, 5, 1]]])  # B=1, H=2, nQ=3
    out = P.plan_items(row, 2, "lpt")
    assert out["bin_ptr"].tolist()[0] == 0 and out["bin_ptr"][-1] == 6
    assert sorted(out["items"].tolist()) == list(range(6))
    assert out["makespan"] == max(out["bin_load"]) == 6
    # item id = (b*H + h)*nQ + q; LPT order: 4(5), 0(3), 2(2), 1(1), 5(1), 3(0)
    assert out["items"].tolist() == [4, 1, 3, 0, 2, 5]


def test_grouped_lpt_hand_example():
    """Heads of loads 12, 3, 9, 6 (3 items each) on 4 bins in 2 groups, worked by hand:
    level 1 puts heads 0 and 1 on group 0 (12, then 3 on the 12/15 tie-free lighter group) and
    heads 2 and 3 on group 1; level 2 runs LPT inside each group; group g's k-th bin is k*2+g."""
    loads = [5, 4, 3, 1, 1, 1, 9, 0, 0, 2, 2, 2]
    bins, bl = P.lpt_grouped(loads, 3, 4, 2)
    assert bins == [[0, 3, 4, 5], [6], [1, 2], [9, 10, 11, 7, 8]]
    assert bl == [8, 9, 7, 6]


def test_grouped_lpt_reduces_to_lpt():
    rng = np.random.default_rng(7)
    loads = rng.integers(0, 20, size=24).tolist()
    assert P.lpt_grouped(loads, 6, 5, 1) == P.lpt(loads, 5)
    assert P.lpt_grouped(loads, 6, 5, 2) == P.lpt(loads, 5)  # 5 bins do not split into 2 groups


# ---- round-based LPT (the device planner's rule) ----

def test_rounds_lpt_page_example_and_hand_cases():
    # db-SP's [8,7,6,5,4] on two machines: round 0 gives 8, 7 to machines 0, 1; round 1 meets
    # loads (8, 7), so 6 goes to machine 1 and 5 to machine 0; round 2 meets a 13/13 tie
    bins, bl = P.lpt_rounds([8, 7, 6, 5, 4], 2)
    assert bins == [[0, 3, 4], [1, 2]] and bl == [17, 13]
    # one job per machine and round: the long job's machine still gets a job in round 1,
    # where plain LPT would have given every short job to machine 1
    bins, bl = P.lpt_rounds([10, 1, 1, 1, 1], 2)
    assert bins == [[0, 3], [1, 2, 4]] and bl == [11, 3]
    assert P.lpt([10, 1, 1, 1, 1], 2)[1] == [10, 4]
    # equal loads: ids ascending within the round, ties between machines to the lower index
    assert P.lpt_rounds([1, 1, 1], 2) == ([[0, 2], [1]], [2, 1])
    # machines ordered ascending by load at the start of a round, not by index
    assert P.lpt_rounds([5, 3, 2, 2], 2) == ([[0, 3], [1, 2]], [7, 5])


def test_rounds_lpt_equals_lpt_in_a_single_round_and_on_equal_loads():
    rng = random.Random(3)
    for _ in range(200):
        m = rng.randint(1, 9)
        loads = [rng.randint(0, 50) for _ in range(rng.randint(0, m))]
        assert P.lpt_rounds(loads, m) == P.lpt(loads, m)
        eq = [7] * rng.randint(0, 30)
        assert P.lpt_rounds(eq, m) == P.lpt(eq, m) == P.naive(eq, m)


def test_rounds_lpt_invariants():
    """Every job once; machine job counts differ by at most one; the spread of machine loads
    never exceeds the longest job (for machines i, j with a_i <= a_j, a round gives i a job
    at least as long as j's, so the new gap is at most max(old gap, the round's longest
    job)); hence makespan <= mean + longest job."""
    rng = random.Random(4)
    for _ in range(300):
        m = rng.randint(1, 12)
        loads = [rng.randint(0, rng.choice([3, 40, 1000])) for _ in range(rng.randint(0, 60))]
        bins, bl = P.lpt_rounds(loads, m)
        assert sorted(j for b in bins for j in b) == list(range(len(loads)))
        counts = [len(b) for b in bins]
        assert max(counts) - min(counts) <= 1
        assert bl == [sum(loads[j] for j in b) for b in bins]
        pmax = max(loads, default=0)
        assert max(bl) - min(bl) <= pmax
        assert max(bl) * m <= sum(loads) + m * pmax
        # within a machine, jobs come in LPT order (one per round)
        for b in bins:
            assert all((-loads[x], x) < (-loads[y], y) for x, y in zip(b, b[1:]))


def test_rounds_lpt_plan_items_and_workload_makespans():
    w = W.make(3)
    row = P.popcount(w.mask, 4)["row"]
    r = P.plan_items(row, 256, "lpt_device")
    assert r["makespan"] == P.plan_items(row, 256, "lpt")["makespan"] == 516
    assert np.array_equal(np.sort(r["items"]), np.arange(row.size))


def test_pair_counts_against_set_unions():
    """Q-block pair loads: the size of the set of KV blocks live in row 2p or row 2p+1, counted
    with Python sets, in total and per contiguous chunk; odd nQ leaves a pair of one row."""
    rng = np.random.default_rng(11)
    for trial in range(40):
        B, H = int(rng.integers(1, 3)), int(rng.integers(1, 4))
        nQ = int(rng.integers(1, 12))
        C = int(rng.choice([1, 2, 3, 4]))
        nK = C * int(rng.integers(1, 5))
        mask = (rng.random((B, H, nQ, nK)) < rng.random()).astype(np.uint8)
        got = P.pair_counts(mask, C)
        striped = P.pair_counts(mask, C, "striped")
        assert np.array_equal(striped["row"], got["row"])
        # a striped chunk holds a slice of every live block: its load is the whole union
        assert all(np.array_equal(striped["crow"][:, :, c, :], got["row"]) for c in range(C))
        nP = (nQ + 1) // 2
        assert got["row"].shape == (B, H, nP) and got["crow"].shape == (B, H, C, nP)
        for b in range(B):
            for h in range(H):
                for p in range(nP):
                    rows = [2 * p] + ([2 * p + 1] if 2 * p + 1 < nQ else [])
                    cols = {j for r in rows for j in range(nK) if mask[b, h, r, j]}
                    assert got["row"][b, h, p] == len(cols)
                    for c in range(C):
                        per = nK // C
                        assert got["crow"][b, h, c, p] == len({j for j in cols if j // per == c})


def test_pair_counts_causal_closed_form_and_bounds():
    """Block-causal mask: pair p covers KV blocks 0 .. 2p+1, so its load is 2p+2 and chunk c of
    width w holds min(w, max(0, 2p+2 - c*w)) of them; in general a pair's load lies between
    the larger and the sum of its two row counts."""
    nQ, C = 64, 4
    mask = np.tril(np.ones((nQ, nQ), np.uint8))[None, None]
    got = P.pair_counts(mask, C)
    p = np.arange(nQ // 2)
    assert np.array_equal(got["row"][0, 0], 2 * p + 2)
    wd = nQ // C
    for c in range(C):
        assert np.array_equal(got["crow"][0, 0, c], np.clip(2 * p + 2 - c * wd, 0, wd))
    w = W.make(4, with_data=False)
    row = P.popcount(w.mask, w.n_chunks)["row"]
    pr = P.pair_counts(w.mask, w.n_chunks)["row"]
    a, b = row[:, :, 0::2], row[:, :, 1::2]
    assert (pr >= np.maximum(a, b)).all() and (pr <= a + b).all()
    # causal workload: LPT over the 1024 pair loads reaches the lower bound of 66560 / 256
    w3 = W.make(3, with_data=False)
    pr3 = P.pair_counts(w3.mask, 4)["row"]
    assert pr3.sum() == 66560
    for order in ("lpt", "lpt_device"):
        assert P.plan_items(pr3, 256, order)["makespan"] == 260
