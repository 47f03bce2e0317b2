"""Oracle: block-mask popcounts, LPT / naive work assignment, brute force, ring step table.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).  Pure Python / numpy
integer arithmetic.

Definitions followed (db-SP post, "load balancing of sparse-attention head
parallelism and sequence parallelism"):

* Scenario 2 bullets: with the block mask's rows as Q-blocks and columns as
  KV-blocks, a Q-block's work is its row sum and a KV-block's its column sum.
* LPT paragraph: repeatedly hand the longest remaining job to the machine that
  is currently least loaded (identical-machines scheduling, makespan
  objective).  The page leaves ties open; the readings used here are
  (i) jobs sorted by load descending, then job id ascending; (ii) among
  equally loaded machines the lowest index wins; (iii) a machine runs its jobs
  in the order they were given to it.  Reading (ii) is the one the page's own
  example needs: [8,7,6,5,4] on two machines must print [8+5+4, 7+6], so the
  final 4 meets a 13/13 tie and goes to machine 0.
* Per-chunk work ("crow"): a chunk is one ring step's KV shard (6D-parallel
  notes, section 2.1).  Contiguous chunk c covers KV blocks
  [c*nK/C, (c+1)*nK/C), so crow counts the row's live blocks in that range.
  Striped chunk c takes tokens j with j mod C == c (section 2.3), so every KV
  block lends block/C tokens to every chunk and crow[c] equals the full row
  count, in units of (block/C)-key groups.
* Ring step table (section 2.3, causal ring skipping): step (r, c) pairs query
  shard r with KV chunk c; query shards follow the same layout rule as the KV
  chunks.  Entry = number of live (query token, key token) pairs.
"""
from __future__ import annotations

import itertools
from typing import Dict, List, Sequence, Tuple

import numpy as np


def popcount(mask: np.ndarray, n_chunks: int, layout: str = "contiguous") -> Dict[str, np.ndarray]:
    """Row, column and per-chunk row counts of a [B, H, nQ, nK] block mask."""
    live = (np.asarray(mask) != 0).astype(np.int64)
    B, H, nQ, nK = live.shape
    row = live.sum(axis=3)
    col = live.sum(axis=2)
    crow = np.zeros((B, H, n_chunks, nQ), dtype=np.int64)
    if layout == "contiguous":
        per = nK // n_chunks
        for c in range(n_chunks):
            crow[:, :, c, :] = live[:, :, :, c * per:(c + 1) * per].sum(axis=3)
    elif layout == "striped":
        for c in range(n_chunks):
            crow[:, :, c, :] = row
    else:
        raise ValueError(layout)
    return {"row": row, "col": col, "crow": crow, "total": int(live.sum())}


def pair_counts(mask: np.ndarray, n_chunks: int, layout: str = "contiguous") -> Dict[str, np.ndarray]:
    """Loads of Q-block pair items on a [B, H, nQ, nK] block mask.

    A pair item p covers Q-blocks 2p and 2p+1 and visits every KV block that is
    live for either of them, so its work is the size of the union of the two
    mask rows (the single-row work of scenario 2 taken over both rows); a lone
    last row of an odd nQ is a pair of one.  Returns the union sizes "row"
    [B, H, nP] and their split over the chunks "crow" [B, H, C, nP]: contiguous
    chunks take their KV-block ranges; every striped chunk holds a slice of each
    live block, so its load is the whole union (as for single rows).
    """
    live = np.asarray(mask) != 0
    B, H, nQ, nK = live.shape
    nP = (nQ + 1) // 2
    union = np.zeros((B, H, nP, nK), dtype=bool)
    for p in range(nP):
        union[:, :, p, :] = live[:, :, 2 * p, :]
        if 2 * p + 1 < nQ:
            union[:, :, p, :] |= live[:, :, 2 * p + 1, :]
    row = union.sum(axis=3).astype(np.int64)
    crow = np.zeros((B, H, n_chunks, nP), dtype=np.int64)
    if layout == "contiguous":
        per = nK // n_chunks
        for c in range(n_chunks):
            crow[:, :, c, :] = union[:, :, :, c * per:(c + 1) * per].sum(axis=3)
    elif layout == "striped":
        for c in range(n_chunks):
            crow[:, :, c, :] = row
    else:
        raise ValueError(layout)
    return {"row": row, "crow": crow}


def lpt(loads: Sequence[int], m: int) -> Tuple[List[List[int]], List[int]]:
    """Longest-processing-time-first greedy onto ``m`` identical machines.

    Returns (per-machine job lists in assignment order, per-machine loads).
    """
    order = sorted(range(len(loads)), key=lambda i: (-int(loads[i]), i))
    bins: List[List[int]] = [[] for _ in range(m)]
    bin_load = [0] * m
    for job in order:
        target = 0
        for b in range(1, m):
            if bin_load[b] < bin_load[target]:
                target = b
        bins[target].append(job)
        bin_load[target] += int(loads[job])
    return bins, bin_load


def lpt_grouped(loads: Sequence[int], items_per_head: int, m: int, groups: int
                ) -> Tuple[List[List[int]], List[int]]:
    """Two-level LPT: heads onto bin groups, then each group's items onto its bins.

    The db-SP post rewards keeping a head's blocks where the head already is
    (its "stay-home" bonus); on one chip the place is the L2 of one XCD, whose
    compute units run the persistent workgroups b with b mod groups == g.  Job
    i = head * items_per_head + q.  Level 1 is LPT of the heads (load = sum of
    their items) onto ``groups`` machines; level 2 is, per group g, LPT of the
    items of g's heads (taken in the order the heads were given to g, then by
    q) onto the m / groups bins of g, whose k-th bin is bin k * groups + g.
    With groups = 1 (or m not a multiple of groups) this is plain LPT.
    """
    n = len(loads)
    if groups <= 1 or m % groups != 0:
        return lpt(loads, m)
    n_heads = n // items_per_head
    head_loads = [sum(int(x) for x in loads[h * items_per_head:(h + 1) * items_per_head]) for h in range(n_heads)]
    head_bins, _ = lpt(head_loads, groups)
    per = m // groups
    bins: List[List[int]] = [[] for _ in range(m)]
    bin_load = [0] * m
    for g in range(groups):
        ids = [h * items_per_head + q for h in head_bins[g] for q in range(items_per_head)]
        local_bins, local_loads = lpt([loads[i] for i in ids], per)
        for k in range(per):
            bins[k * groups + g] = [ids[j] for j in local_bins[k]]
            bin_load[k * groups + g] = local_loads[k]
    return bins, bin_load


def lpt_rounds(loads: Sequence[int], m: int) -> Tuple[List[List[int]], List[int]]:
    """Round-based LPT: the jobs in LPT order are handed out m at a time.

    A parallel form of the LPT paragraph's greedy (one sort per round instead of
    one least-loaded search per job).  Jobs are taken in the LPT order (load
    descending, id ascending).  In each round the next m jobs go to the machines
    ordered by their load at the start of the round (ascending, lower index
    first on equal loads): the round's j-th job to the j-th machine, so the
    round's longest job meets the least-loaded machine.  Every machine gets one
    job per round, except in a last, partial round.  With at most m jobs, or a
    single round, this is exactly LPT.
    """
    order = sorted(range(len(loads)), key=lambda i: (-int(loads[i]), i))
    bins: List[List[int]] = [[] for _ in range(m)]
    bin_load = [0] * m
    for r0 in range(0, len(order), m):
        machines = sorted(range(m), key=lambda b: (bin_load[b], b))
        for job, b in zip(order[r0:r0 + m], machines):
            bins[b].append(job)
            bin_load[b] += int(loads[job])
    return bins, bin_load


def lpt_order(loads: Sequence[int]) -> List[int]:
    """The jobs in LPT order: load descending, then job id ascending (reading (i) above).

    The queue of the LPT paragraph's greedy in its list-scheduling form: whenever a machine
    becomes free it takes the next job of this list.  With run times equal to the loads,
    the machine that becomes free first is the least-loaded one, so the form gives ``lpt``'s
    assignment (``list_schedule`` below shows it on given run times).
    """
    return sorted(range(len(loads)), key=lambda i: (-int(loads[i]), i))


def list_schedule(order: Sequence[int], times: Sequence[float], m: int) -> List[List[int]]:
    """Runs the jobs of ``order`` on m machines, each free machine taking the next job.

    ``times[j]`` is job j's run time.  Among machines free at the same moment the lowest
    index takes the job first (reading (ii) above).  Returns each machine's jobs in order.
    """
    free_at = [0.0] * m
    bins: List[List[int]] = [[] for _ in range(m)]
    for job in order:
        b = min(range(m), key=lambda k: (free_at[k], k))
        bins[b].append(job)
        free_at[b] += float(times[job])
    return bins


def naive(loads: Sequence[int], m: int) -> Tuple[List[List[int]], List[int]]:
    """Round-robin in job-id order: job i runs on machine i mod m."""
    bins: List[List[int]] = [[] for _ in range(m)]
    bin_load = [0] * m
    for i, p in enumerate(loads):
        bins[i % m].append(i)
        bin_load[i % m] += int(p)
    return bins, bin_load


def brute_force_makespan(loads: Sequence[int], m: int) -> Tuple[int, Tuple[int, ...]]:
    """Optimal makespan by trying every one of the m**n assignments (tiny inputs only)."""
    best, best_assign = None, None
    for assign in itertools.product(range(m), repeat=len(loads)):
        tot = [0] * m
        for job, b in enumerate(assign):
            tot[b] += int(loads[job])
        span = max(tot)
        if best is None or span < best:
            best, best_assign = span, assign
    return best, best_assign


def plan_items(row_loads: np.ndarray, m: int, order: str = "lpt", groups: int = 1) -> Dict[str, np.ndarray]:
    """Assign every (b, h, q) item (id = (b*H + h)*nQ + q, load = row count) to m bins.

    ``order``: "lpt", "naive", "lpt_device" (``lpt_rounds``) or "lpt_xcd"
    (``lpt_grouped`` with the heads of ``row_loads`` [B, H, nQ] and ``groups``
    bin groups); "lpt_dynamic" makes the bins of "lpt_device" and adds ``queue``,
    the items in LPT order.  Returns ``items`` (all
    bins' lists concatenated), ``bin_ptr`` (m + 1 offsets), ``bin_load`` and
    ``makespan``.
    """
    row_loads = np.asarray(row_loads, dtype=np.int64)
    loads = row_loads.reshape(-1).tolist()
    if order == "lpt_xcd":
        bins, bin_load = lpt_grouped(loads, row_loads.shape[-1], m, groups)
    else:
        bins, bin_load = {"lpt": lpt, "naive": naive, "lpt_device": lpt_rounds,
                          "lpt_dynamic": lpt_rounds}[order](loads, m)
    items, ptr = [], [0]
    for b in bins:
        items.extend(b)
        ptr.append(len(items))
    out = {"items": np.array(items, dtype=np.int64), "bin_ptr": np.array(ptr, dtype=np.int64),
           "bin_load": np.array(bin_load, dtype=np.int64), "makespan": int(max(bin_load))}
    if order == "lpt_dynamic":
        out["queue"] = np.array(lpt_order(loads), dtype=np.int64)
    return out


def _tokens_per_block_in_part(S: int, block: int, n_parts: int, layout: str) -> np.ndarray:
    """[n_parts, nBlocks] count of a block's tokens that fall in each shard / chunk."""
    nb = -(-S // block)
    cnt = np.zeros((n_parts, nb), dtype=np.int64)
    per = nb // n_parts
    for t in range(S):
        blk = t // block
        part = (blk // per) if layout == "contiguous" else (t % n_parts)
        cnt[part, blk] += 1
    return cnt


def step_table(mask: np.ndarray, S: int, block: int, n_chunks: int, layout: str) -> np.ndarray:
    """[B, H, C, C] live token pairs of ring step (query shard r, KV chunk c)."""
    live = (np.asarray(mask) != 0).astype(np.int64)
    cnt = _tokens_per_block_in_part(S, block, n_chunks, layout)
    # pairs[r, c] = sum_i sum_j cnt[r, i] * live[i, j] * cnt[c, j]
    return np.einsum("ri,bhij,cj->bhrc", cnt, live, cnt)
