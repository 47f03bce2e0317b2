"""Benchmark of the block-sparse attention hot path on one MI355X.

One step = one pass of the whole path over one batch of the causal long-sequence
workload (B1 H16 S16384 d128, block 128, lower-triangular block mask, KV in 4 contiguous
chunks, one bin per compute unit):

  1. sparse_attn_plan: GPU popcount of the mask and the work lists, by default with the
     device planner (round-based LPT made on the GPU; --order lpt_dynamic: the same plan's
     LPT queue, taken by the attention kernel's workgroups at run time, one counter per XCD;
     lpt_xcd / lpt / naive plan on the host instead).  The mask is a runtime input, so every step re-plans, on a
     side stream; the forward call waits for the plan's event;
  2. sparse_attn_fwd in partial mode over chunks [0, 4): one (O, m, l) partial per chunk;
  3. chunk_merge: online-softmax merge of the 4 partials into O (bf16).

value = live-block FLOP per step (4 * 128^3 per live tile) / measured step time.

The untimed extras also run the token top-k path on its own workload (B1 H16 n32768 d128,
rank-32 indexer, top-k 512, causal): the TOPK plan (projections + importance + per-query
top-k) and the gather attention over the selected keys, reported as times and rates.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--mode merged|fused]
       [--workload causal|video|skewed|tiny] [--layout contiguous|striped] [--no-cpu-baseline]
       [--no-extras] [--no-workloads] [--no-topk] [--calibrate-copy MiB]

Before the W warmup steps the step is repeated, untimed, for --settle seconds (0.25 by default):
from idle the GPU needs about 15 steps to reach its sustained clock.  Each step's plan is
destroyed inside the timed loop right after the next step is issued (the
library returns its buffers to a cache and reuses them once the kernels that read them are done,
so no step allocates or synchronises).  The untimed extras also time the other block-sparse
workloads: the causal one in the other chunk layout, the video and the skewed workload, each as a
whole step and in LPT and round-robin order with measured per-CU balance.
Prints one JSON line.  Only one GPU is used: --gpus > 1 exits with a message.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

METRIC = "live-block attention TFLOP/s + % bf16 MFMA peak; per-CU max/mean work"
PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, published
HBM_PEAK_GBS = 8000.0
WORKLOADS = {"tiny": 1, "video": 2, "causal": 3, "skewed": 4}
PAIR_OVERHEAD_MAX = 1.05  # Q-block pairs when the union tiles they compute exceed the live tiles by at most 5%
KERNEL_SOURCES = ["sparse_mask_load_amd/csrc/attn_bf16.hip", "sparse_mask_load_amd/csrc/kernel_common.h",
                  "sparse_mask_load_amd/csrc/internal.h"]


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def read_counter_traffic(workload: str):
    """HBM bytes per attention launch from the committed rocprofv3 counter summary.

    Returns None when no summary exists or the kernel source changed since the counters
    were taken (the summary records the source hash it was made with).
    """
    path = os.path.join(ROOT, "profiles", f"attn_bf16_{workload}_hbm_counters.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_hash = re.search(r"kernel source hash:\s*`?([0-9a-f]+)", text)
    m_bytes = re.search(r"HBM bytes per launch \(scaled\):\s*([0-9.eE+]+)", text)
    if not m_hash or not m_bytes or m_hash.group(1) != kernel_source_hash():
        return None
    return float(m_bytes.group(1))


def cpu_baseline(w, n_heads: int):
    """Time the CPU oracle (as it stands) on a bounded sample of the workload."""
    from threadpoolctl import threadpool_info

    from oracle import attention as A
    from oracle import plan as P

    hs = slice(0, n_heads)
    t0 = time.perf_counter()
    cnt = P.popcount(w.mask, w.n_chunks, w.layout)
    P.plan_items(cnt["row"], 256, "lpt")
    parts = [A.chunk_partial(w.q[:, hs], w.k[:, hs], w.v[:, hs], w.mask[:, hs], w.block, w.n_chunks, w.layout, c)
             for c in range(w.n_chunks)]
    A.merge(parts)
    dt = time.perf_counter() - t0
    flop = 4.0 * w.block * w.block * w.D * int(cnt["row"][:, hs].sum())
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    return {"value": flop / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": f"fp64 numpy oracle on heads 0-{n_heads - 1} of {w.H} (all their live tiles, "
                      f"{w.n_chunks} chunk partials + merge) plus popcount and LPT of the whole mask; "
                      f"{dt:.1f} s wall"}


def peak_clock_mhz(device: int):
    """The GPU's peak engine clock from the HIP runtime (hipDeviceAttributeClockRate, in kHz), or None."""
    import ctypes
    try:
        hip = ctypes.CDLL("libamdhip64.so")
        khz = ctypes.c_int(0)
        hip_device_attribute_clock_rate = 5  # position of hipDeviceAttributeClockRate in hipDeviceAttribute_t
        if hip.hipDeviceGetAttribute(ctypes.byref(khz), hip_device_attribute_clock_rate, device) != 0:
            return None
        return khz.value // 1000 or None
    except OSError:
        return None


def per_cu_balance(trace: np.ndarray):
    """Busy time per compute unit (hardware XCC / SE / CU id of each item) and per workgroup."""
    start, end, hw, binitem = trace[:, 0], trace[:, 1], trace[:, 2], trace[:, 3]
    busy = (end - start).astype(np.float64)
    xcc = hw >> 32
    cu_key = xcc * 256 + ((hw & 0xFFFFFFFF) >> 8 & 0xFF)
    per_cu = {}
    for k, b in zip(cu_key.tolist(), busy.tolist()):
        per_cu[k] = per_cu.get(k, 0.0) + b
    per_bin = {}
    for k, b in zip((binitem >> 32).tolist(), busy.tolist()):
        per_bin[k] = per_bin.get(k, 0.0) + b
    cu = np.array(list(per_cu.values()))
    bins = np.array(list(per_bin.values()))
    return {"cus_used": int(len(cu)), "measured_cu_max_over_mean": float(cu.max() / cu.mean()),
            "measured_bin_max_over_mean": float(bins.max() / bins.mean())}


def topk_path(bd, W, torch, dev, reps: int = 5) -> dict:
    """Times the top-k path (indexer + selection, gather attention) on the 16x32768 workload."""
    w = W.make(5)
    q, k, v = (torch.from_numpy(x).to(dev, torch.bfloat16) for x in (w.q, w.k, w.v))
    wq, wk = (torch.from_numpy(np.ascontiguousarray(x)).to(dev, torch.bfloat16) for x in (w.wq, w.wk))
    prob = bd.make_problem(q, 0, 1, "contiguous")
    out = torch.empty_like(q)
    stream = torch.cuda.current_stream()

    def plan():
        return bd.sparse_attn_plan(prob, "topk", q=q, k=k, wq=wq, wk=wk, rank=w.rank, top_k=w.top_k, causal=True)

    p = plan()
    bd.sparse_attn_fwd(p, q, k, v, 0, 1, o=out)
    torch.cuda.synchronize()
    info = bd.sparse_attn_plan_info(p)
    e = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    t_idx, t_att = [], []
    for _ in range(reps):
        e[0].record(stream)
        p2 = plan()
        e[1].record(stream)
        e[2].record(stream)
        bd.sparse_attn_fwd(p2, q, k, v, 0, 1, o=out)
        e[3].record(stream)
        torch.cuda.synchronize()
        p2.close()
        t_idx.append(e[0].elapsed_time(e[1]))
        t_att.append(e[2].elapsed_time(e[3]))
    p.close()
    B, H, S, D = q.shape
    cand = B * H * S * (S + 1) // 2  # causal candidate pairs
    pairs = int(info["total_live"])
    idx_ms, att_ms = float(np.median(t_idx)), float(np.median(t_att))
    return {
        "workload": f"top-k token-sparse attention B{B} H{H} n{S} d{D}, rank {w.rank} indexer, top-k {w.top_k}, causal",
        "indexer_ms": round(idx_ms, 4), "candidates": cand,
        "indexer_gcand_per_s": round(cand / idx_ms / 1e6, 1),
        "indexer_mfma_tflops": round(2.0 * w.rank * cand / idx_ms / 1e9, 2),
        "gather_attention_ms": round(att_ms, 4), "selected_pairs": pairs,
        "gather_attention_tflops": round(4.0 * D * pairs / att_ms / 1e9, 2),
        "gather_kv_gbs": round(2 * D * 2 * pairs / att_ms / 1e6, 1),
        "path_ms": round(idx_ms + att_ms, 4),
    }


class WorkloadRun:
    """One block-sparse workload resident on the GPU: Q, K, V, mask, chunk partials, output."""

    def __init__(self, bd, torch, dev, w, layout=None, q_pairs="auto"):
        self.bd, self.torch, self.w = bd, torch, w
        dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
        self.q, self.k, self.v = (torch.from_numpy(x).to(dev, dt) for x in (w.q, w.k, w.v))
        self.mask = torch.from_numpy(w.mask).to(dev)
        self.layout = layout or w.layout
        B, H, S, D = self.q.shape
        C = w.n_chunks
        self.B, self.H, self.S, self.D, self.C = B, H, S, D, C
        self.prob_single = bd.make_problem(self.q, w.block, C, self.layout)
        # Q-block pair items where the kernel has them and adjacent mask rows share their tiles:
        # the pairs' union tiles (what the pair kernel computes) against the live tiles
        self.q_pairs, self.pair_overhead = False, None
        if q_pairs != "off" and w.dtype == "bf16" and w.block == 128 and S % 128 == 0:
            prob_p = bd.make_problem(self.q, w.block, C, self.layout, q_pairs=True)
            p = bd.sparse_attn_plan(prob_p, "block", mask=self.mask, order="lpt")
            info = bd.sparse_attn_plan_info(p)
            p.close()
            self.pair_overhead = 2.0 * info["load_sum"] / max(1, info["total_live"])
            self.q_pairs = q_pairs == "on" or self.pair_overhead <= PAIR_OVERHEAD_MAX
        elif q_pairs == "on":
            raise SystemExit("--q-pairs on needs a bf16 workload with block 128 and S % 128 == 0")
        self.prob = bd.make_problem(self.q, w.block, C, self.layout, q_pairs=self.q_pairs)
        self.o_part = torch.empty((C, B, H, S, D), dtype=torch.float32, device=dev)
        self.m_part = torch.empty((C, B, H, S), dtype=torch.float32, device=dev)
        self.l_part = torch.empty((C, B, H, S), dtype=torch.float32, device=dev)
        self.out = torch.empty_like(self.q)
        self.rows = B * H * S

    def plan(self, order, bins=0, stream=None, prob=None):
        return self.bd.sparse_attn_plan(prob or self.prob, "block", mask=self.mask, order=order, num_bins=bins,
                                        stream=stream)

    def fwd_partial(self, plan):
        self.bd.sparse_attn_fwd(plan, self.q, self.k, self.v, 0, self.C, o_part=self.o_part, m_part=self.m_part,
                                l_part=self.l_part)

    def fwd_fused(self, plan, trace=None):
        self.bd.sparse_attn_fwd(plan, self.q, self.k, self.v, 0, self.C, o=self.out, trace=trace)

    def merge(self):
        C = self.C
        self.bd.chunk_merge([self.o_part[c] for c in range(C)], [self.m_part[c] for c in range(C)],
                            [self.l_part[c] for c in range(C)], self.rows, self.D, self.out, self.w.dtype)

    def merge_bytes(self):
        """HBM bytes the merge moves: m and l of every part, O of the parts whose row has a key
        (the merge skips O of empty parts), and the output written once."""
        nonempty = int(self.torch.isfinite(self.m_part).sum().item())
        out_b = 2 if self.w.dtype == "bf16" else 4
        return self.rows * self.C * 8 + nonempty * self.D * 4 + self.rows * self.D * out_b

    def flop(self, total_live):
        return 4.0 * self.w.block * self.w.block * self.D * total_live

    def kernel_name(self):
        """The attention kernel the forward call launches for this workload."""
        if self.w.dtype != "bf16":
            return "attn_f32_kernel"
        if self.q_pairs:
            return "attn_bf16_pair_kernel"
        if self.w.block == 128 and (self.layout == "striped" or self.S % 128 == 0):
            return "attn_bf16_pipe_kernel"
        return "attn_bf16_kernel"

    def timed(self, fn, reps):
        """Mean time of fn() over reps launches (HIP events on the current stream), after about
        30 ms of untimed launches (at least three): right after the timed partial-mode loop the
        first dozen full-mode launches run about 10% slower than later ones."""
        torch = self.torch
        stream = torch.cuda.current_stream()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        fn()
        torch.cuda.synchronize()
        once = time.perf_counter() - t0
        for _ in range(min(50, max(3, int(0.03 / max(once, 1e-6))))):
            fn()
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    def steps(self, order, n, warmup=2, settle=0.1):
        """ms per whole step (plan on a side stream, partial forward, merge), the previous step's plan
        destroyed inside the loop, and the forward's mean time from HIP events."""
        torch = self.torch
        stream = torch.cuda.current_stream()
        plan_stream = torch.cuda.Stream()
        fwd = []

        def one(record):
            plan = self.plan(order, stream=plan_stream)
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            self.fwd_partial(plan)
            e1.record(stream)
            self.merge()
            if record:
                fwd.append((e0, e1))
            return plan

        prev = None
        t_settle = time.perf_counter()
        while time.perf_counter() - t_settle < settle:
            p = one(False)
            if prev is not None:
                prev.close()
            prev = p
            torch.cuda.synchronize()
        for _ in range(warmup):
            p = one(False)
            if prev is not None:
                prev.close()
            prev = p
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(n):
            p = one(True)
            prev.close()  # the previous step's plan: its buffers are reused once its kernels are done
            prev = p
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        prev.close()
        return (t1 - t0) * 1e3 / n, float(np.mean([a.elapsed_time(b) for a, b in fwd]))

    def ring_steps(self, order, reps):
        """The ring emulation: one forward launch per KV chunk, each over that chunk's own LPT list
        (the per-step greedy), then the merge.  Per chunk: its time, the planned bin max/mean of
        its own list and of the full-range list carrying the same chunk's loads (one assignment
        reused for every step), and the measured per-CU balance."""
        bd, torch = self.bd, self.torch
        p = self.plan(order)
        info = bd.sparse_attn_plan_info(p)
        m, n, C = info["num_bins"], info["n_items"], self.C
        nI = (info["nQ"] + 1) // 2 if self.q_pairs else info["nQ"]
        items0 = bd.sparse_attn_plan_copy(p, bd.SA_PLAN_ITEMS, n)
        ptr0 = bd.sparse_attn_plan_copy(p, bd.SA_PLAN_BIN_PTR, m + 1)
        crow = bd.sparse_attn_plan_copy(p, bd.SA_PLAN_PAIR_CROW if self.q_pairs else bd.SA_PLAN_CROW,
                                        self.B * self.H * C * nI).reshape(self.B * self.H, C, nI)
        bin_of = np.repeat(np.arange(m), np.diff(ptr0))
        chunks = []
        for c in range(C):
            own = bd.sparse_attn_plan_copy(p, bd.SA_PLAN_BIN_LOAD, m, chunk=c)
            full = np.bincount(bin_of, weights=crow[items0 // nI, c, items0 % nI], minlength=m)
            trace = torch.zeros((n, 4), dtype=torch.int64, device=self.q.device)
            args = dict(o_part=self.o_part[c], m_part=self.m_part[c], l_part=self.l_part[c])
            bd.sparse_attn_fwd(p, self.q, self.k, self.v, c, c + 1, trace=trace, **args)
            torch.cuda.synchronize()
            bal = per_cu_balance(trace.cpu().numpy())
            ms = self.timed(lambda: bd.sparse_attn_fwd(p, self.q, self.k, self.v, c, c + 1, **args), reps)
            chunks.append({"chunk": c, "fwd_ms": round(ms, 4), "live_tiles": int(crow[:, c, :].sum()),
                           "planned_bin_max_over_mean_own_list": round(float(own.max() / own.mean()), 4),
                           "planned_bin_max_over_mean_full_list": round(float(full.max() / full.mean()), 4),
                           "measured_cu_max_over_mean": round(bal["measured_cu_max_over_mean"], 4)})

        def ring():
            for c in range(C):
                bd.sparse_attn_fwd(p, self.q, self.k, self.v, c, c + 1, o_part=self.o_part[c],
                                   m_part=self.m_part[c], l_part=self.l_part[c])
            self.merge()
        step = self.timed(ring, reps)
        p.close()
        return {"per_chunk": chunks, "fwd_ms_sum": round(sum(x["fwd_ms"] for x in chunks), 4),
                "ring_step_ms": round(step, 4)}

    def order_summary(self, order, reps):
        """Fused and partial forward time of one work order, its planned and measured per-CU balance."""
        bd, torch = self.bd, self.torch
        p = self.plan(order)
        info = bd.sparse_attn_plan_info(p)
        bl = bd.sparse_attn_plan_copy(p, bd.SA_PLAN_BIN_LOAD, info["num_bins"])
        trace = torch.zeros((info["n_items"], 4), dtype=torch.int64, device=self.q.device)
        self.fwd_fused(p, trace=trace)
        torch.cuda.synchronize()
        bal = per_cu_balance(trace.cpu().numpy())
        fused = self.timed(lambda: self.fwd_fused(p), reps)
        partial = self.timed(lambda: self.fwd_partial(p), reps)
        p.close()
        return {"fwd_fused_ms": round(fused, 4), "fwd_partial_ms": round(partial, 4),
                "fused_tflops": round(self.flop(info["total_live"]) / fused / 1e9, 2),
                "planned_makespan_tiles": info["makespan"], "lower_bound_tiles": info["lower_bound"],
                "planned_bin_max_over_mean": round(float(bl.max() / bl.mean()), 4),
                "measured_cu_max_over_mean": round(bal["measured_cu_max_over_mean"], 4)}


def workload_summary(bd, W, torch, dev, cfg, layout="contiguous", steps=10, reps=5, ring=False):
    """Untimed extra: another workload's whole step (device plan, partial forward over every chunk,
    merge) and its forward in device-planned LPT, host LPT and round-robin order; with `ring`,
    also the one-launch-per-chunk ring emulation."""
    w = W.make(cfg, layout=layout)
    run = WorkloadRun(bd, torch, dev, w)
    items = "Q-block pairs" if run.q_pairs else "Q-blocks"
    p = run.plan("lpt_device")
    info = bd.sparse_attn_plan_info(p)
    p.close()
    flop = run.flop(info["total_live"])
    step_ms, fwd_ms = run.steps("lpt_device", steps)
    merge_ms = run.timed(run.merge, reps)
    out = {"workload": f"{w.name} B{run.B} H{run.H} S{run.S} d{run.D} block {w.block}, {run.C} {layout} chunks, "
                       f"work items: {items}",
           "kernel": run.kernel_name(), "pair_overhead": run.pair_overhead,
           "live_tiles": info["total_live"], "flop": flop,
           "ms_per_step": round(step_ms, 4), "step_tflops": round(flop / step_ms / 1e9, 2),
           "step_pct_bf16_peak": round(100 * flop / step_ms / 1e9 / PEAK_BF16_TFLOPS, 2),
           "fwd_partial_ms": round(fwd_ms, 4), "fwd_partial_tflops": round(flop / fwd_ms / 1e9, 2),
           "merge_ms": round(merge_ms, 4), "merge_gbs": round(run.merge_bytes() / merge_ms / 1e6, 1),
           "by_order": {o: run.order_summary(o, reps) for o in ("lpt_dynamic", "lpt_device", "lpt", "naive")}}
    if ring:
        out["ring_steps"] = run.ring_steps("lpt_device", reps)
    del run
    torch.cuda.empty_cache()
    return out


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--settle", type=float, default=0.25,
                    help="seconds of untimed steps before the warmup steps (the GPU's clock settles)")
    ap.add_argument("--workload", choices=sorted(WORKLOADS), default="causal")
    ap.add_argument("--layout", choices=["contiguous", "striped"], default="contiguous",
                    help="KV chunk layout: contiguous blocks, or striped (token i in chunk i mod C)")
    ap.add_argument("--mode", choices=["merged", "fused"], default="merged",
                    help="merged: partial chunks + chunk_merge (default); fused: chunks folded in-kernel")
    ap.add_argument("--order", choices=["lpt_xcd", "lpt", "naive", "lpt_device", "lpt_dynamic"], default="lpt_device",
                    help="work order: two-level LPT (heads to XCDs, then Q-blocks), one-level LPT, round-robin, "
                         "round-based LPT made on the GPU, or the GPU-made LPT queue taken at run time")
    ap.add_argument("--bins", type=int, default=0, help="persistent workgroups (0: one per resident slot)")
    ap.add_argument("--q-pairs", choices=["auto", "on", "off"], default="auto",
                    help="work items of two adjacent Q-blocks (auto: where their union tiles exceed the live "
                         f"tiles by at most {round(100 * (PAIR_OVERHEAD_MAX - 1))}%%)")
    ap.add_argument("--cpu-heads", type=int, default=12, help="heads of the oracle's timed sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true", help="skip the untimed breakdown runs")
    ap.add_argument("--no-topk", action="store_true", help="skip the token top-k path measurement")
    ap.add_argument("--no-workloads", action="store_true",
                    help="skip the other block-sparse workloads (striped causal, video, skewed)")
    ap.add_argument("--topk-only", action="store_true",
                    help="diagnostic: run only the token top-k path (for profiling its kernels) and print its "
                         "figures; no block-sparse step, no metric")
    ap.add_argument("--calibrate-copy", type=int, default=0,
                    help="also run a plain device copy of this many MiB (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (this library does not shard); got --gpus {args.gpus}",
              file=sys.stderr)
        return 2

    import torch

    from sparse_mask_load_amd import binding as bd
    from sparse_mask_load_amd import workloads as W

    if not os.path.exists(bd.LIB_PATH):
        from sparse_mask_load_amd import build as _b
        _b.build()
    bd.lib()
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    if args.topk_only:
        print(json.dumps({"topk_path": topk_path(bd, W, torch, dev)}), flush=True)
        return 0

    w = W.make(WORKLOADS[args.workload], layout=args.layout)
    run = WorkloadRun(bd, torch, dev, w, q_pairs=args.q_pairs)
    q, k, v, mask, out = run.q, run.k, run.v, run.mask, run.out
    B, H, S, D, C = run.B, run.H, run.S, run.D, run.C
    prob = run.prob
    stream = torch.cuda.current_stream()
    # the plan of a step is built on a side stream: its host part (counts, LPT, uploads) then
    # overlaps the previous step's attention on the main stream, and the forward call waits
    # for the plan's uploads by itself
    plan_stream = torch.cuda.Stream()
    fwd_events = []

    def step(record: bool):
        plan = run.plan(args.order, args.bins, stream=plan_stream)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        if args.mode == "merged":
            run.fwd_partial(plan)
            e1.record(stream)
            run.merge()
        else:
            run.fwd_fused(plan)
            e1.record(stream)
        if record:
            fwd_events.append((e0, e1))
        return plan

    prev = None
    # untimed: bring the GPU to its sustained clock (it takes about 15 steps from idle), then
    # the W warmup steps
    t_settle = time.perf_counter()
    while time.perf_counter() - t_settle < args.settle:
        p = step(False)
        if prev is not None:
            prev.close()
        prev = p
        torch.cuda.synchronize()
    for _ in range(args.warmup):
        p = step(False)
        if prev is not None:
            prev.close()
        prev = p
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        p = step(True)
        if prev is not None:
            prev.close()  # step i-1's plan, inside the timed loop (its buffers return to the cache)
        prev = p
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    prev.close()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    kernel_ms = float(np.mean([a.elapsed_time(b) for a, b in fwd_events]))

    plan = run.plan(args.order, args.bins)
    info = bd.sparse_attn_plan_info(plan)
    flop = run.flop(info["total_live"])
    value = flop / (ms_per_step * 1e-3) / 1e12
    achieved = flop / (kernel_ms * 1e-3) / 1e12
    bin_load = bd.sparse_attn_plan_copy(plan, bd.SA_PLAN_BIN_LOAD, info["num_bins"])
    traffic_key = args.workload if args.layout == "contiguous" else f"{args.workload}_{args.layout}"

    result = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": f"{w.name} block-sparse MHA B{B} H{H} S{S} d{D} block {w.block}, "
                               f"{C} {args.layout} KV chunks {'merged by chunk_merge' if args.mode == 'merged' else 'folded in-kernel'}, "
                               f"work items: {'Q-block pairs' if run.q_pairs else 'Q-blocks'}, "
                               f"{ {'lpt_xcd': 'two-level LPT (heads to XCDs, then Q-blocks)', 'lpt': 'LPT', 'naive': 'round-robin', 'lpt_device': 'round-based LPT made on the GPU', 'lpt_dynamic': 'LPT queue made on the GPU, taken at run time'}[args.order]} over {info['num_bins']} bins",
                   "B": B, "H": H, "S": S, "D": D, "block": w.block, "n_chunks": C, "layout": args.layout,
                   "mask": {"tiny": "Bernoulli(0.5)+diag", "video": "frame band / Bernoulli",
                            "causal": "block lower-triangular", "skewed": "Zipf(1.2) rows"}[args.workload],
                   "live_tiles": info["total_live"], "mode": args.mode, "order": args.order,
                   "q_pairs": run.q_pairs},
        "pct_bf16_peak_step": round(100.0 * value / PEAK_BF16_TFLOPS, 2),
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": read_counter_traffic(traffic_key),
                     "kernel": run.kernel_name(), "kernel_ms": round(kernel_ms, 4),
                     "kernel_source_hash": kernel_source_hash()},
        "per_cu_work": {"planned_bin_max_over_mean": round(float(bin_load.max() / bin_load.mean()), 4),
                        "planned_makespan_tiles": info["makespan"], "lower_bound_tiles": info["lower_bound"]},
    }

    if not args.no_extras:
        reps = 10
        # per-CU busy time from the in-kernel trace (one untimed launch)
        trace = torch.zeros((info["n_items"], 4), dtype=torch.int64, device=dev)
        run.fwd_fused(plan, trace=trace)
        torch.cuda.synchronize()
        result["per_cu_work"].update(per_cu_balance(trace.cpu().numpy()))
        fused_ms = run.timed(lambda: run.fwd_fused(plan), reps)
        merge_ms = run.timed(run.merge, reps)
        merge_gbs = run.merge_bytes() / merge_ms / 1e6
        t_plan = time.perf_counter()
        for _ in range(reps):  # host planner (waits for the counts, LPT on the host)
            run.plan("lpt_xcd").close()
        plan_host_ms = (time.perf_counter() - t_plan) * 1e3 / reps
        # device planner: host cost of the call (it returns without waiting) and its GPU time
        t_plan = time.perf_counter()
        dplans = [run.plan("lpt_device") for _ in range(reps)]
        plan_device_call_ms = (time.perf_counter() - t_plan) * 1e3 / reps
        torch.cuda.synchronize()
        for p_d in dplans:
            p_d.close()
        gpu_ms = []
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        for _ in range(reps):  # device-side latency: mask copy, popcount and the planning kernel
            e0.record(stream)
            p_d = run.plan("lpt_device", stream=stream)
            e1.record(stream)
            torch.cuda.synchronize()
            gpu_ms.append(e0.elapsed_time(e1))
            p_d.close()
        plan_device_gpu_ms = float(np.median(gpu_ms))
        # whole steps with the other planner (same loop as the timed one)
        other_order = "lpt_xcd" if args.order == "lpt_device" else "lpt_device"
        step_other_ms, _ = run.steps(other_order, args.steps)
        # persistent orders over one bin per resident workgroup, then one item per workgroup
        # (a plain grid that the hardware dispatches as compute units free up), in id order
        # and in LPT order
        alt_ms = {}
        n_items = info["n_items"]
        alts = [(o_, o_, 0) for o_ in ("naive", "lpt", "lpt_xcd", "lpt_device", "lpt_dynamic")]
        alts += [("grid_id_order", "naive", n_items), ("grid_lpt_order", "lpt", n_items)]
        for alt, alt_order, alt_bins in alts:
            p_alt = run.plan(alt_order, alt_bins)
            alt_ms[alt] = (run.timed(lambda: run.fwd_fused(p_alt), reps), bd.sparse_attn_plan_info(p_alt))
            p_alt.close()
        # the same mask with token-level causality inside the live tiles
        p_tc = run.plan(args.order, prob=bd.make_problem(q, w.block, C, args.layout, token_causal=True,
                                                         q_pairs=run.q_pairs))
        tc_ms = run.timed(lambda: run.fwd_fused(p_tc), reps)
        p_tc.close()
        # the partial-mode forward with cold caches: a 512 MiB write first evicts the L2s and
        # the Infinity Cache (256 MiB), so Q, K and V come from HBM (median of 3)
        evict = torch.empty(128 << 20, dtype=torch.float32, device=dev)
        cold = []
        for _ in range(3):
            evict.fill_(1.0)
            e0.record(stream)
            run.fwd_partial(plan)
            e1.record(stream)
            torch.cuda.synchronize()
            cold.append(e0.elapsed_time(e1))
        del evict
        partial_cold_ms = float(np.median(cold))
        # measured per-CU balance of the round-robin order, beside the step's planner above
        p_naive = run.plan("naive")
        tr_naive = torch.zeros((info["n_items"], 4), dtype=torch.int64, device=dev)
        run.fwd_fused(p_naive, trace=tr_naive)
        torch.cuda.synchronize()
        naive_balance = per_cu_balance(tr_naive.cpu().numpy())
        p_naive.close()
        # the ring emulation: one launch per chunk over its own list (per-step LPT), then the merge
        ring = run.ring_steps(args.order, reps)
        # the same step's forward with single Q-block items (when the step uses pairs)
        single = {}
        if run.q_pairs:
            p_s = run.plan(args.order, prob=run.prob_single)
            single = {"fwd_partial_single_items_ms": round(run.timed(lambda: run.fwd_partial(p_s), reps), 4),
                      "fwd_fused_single_items_ms": round(run.timed(lambda: run.fwd_fused(p_s), reps), 4)}
            p_s.close()
        props = torch.cuda.get_device_properties(dev)
        result["device"] = {"name": props.name, "arch": getattr(props, "gcnArchName", None),
                            "compute_units": props.multi_processor_count, "peak_clock_mhz": peak_clock_mhz(dev.index or 0)}
        result["per_cu_work"]["naive_measured_cu_max_over_mean"] = naive_balance["measured_cu_max_over_mean"]
        result["breakdown"] = {
            "plan_host_ms": round(plan_host_ms, 4), "fwd_partial_ms": round(kernel_ms, 4),
            "fwd_partial_cold_ms": round(partial_cold_ms, 4),
            "fwd_fused_ms": round(fused_ms, 4), "fused_tflops": round(flop / fused_ms / 1e9, 2),
            "fused_pct_bf16_peak": round(100 * flop / fused_ms / 1e9 / PEAK_BF16_TFLOPS, 2),
            "merge_ms": round(merge_ms, 4), "merge_gbs": round(merge_gbs, 1),
            "merge_frac_hbm_peak": round(merge_gbs / HBM_PEAK_GBS, 4),
            "fwd_fused_ms_by_order": {o: round(t, 4) for o, (t, _) in alt_ms.items()},
            "makespan_tiles_by_order": {o: i["makespan"] for o, (_, i) in alt_ms.items()},
            "xcd_groups": alt_ms["lpt_xcd"][1]["groups"],
            "fwd_fused_token_causal_ms": round(tc_ms, 4),
            "plan_device_call_ms": round(plan_device_call_ms, 4), "plan_device_gpu_ms": round(plan_device_gpu_ms, 4),
            "ms_per_step_by_planner": {args.order: round(ms_per_step, 4), other_order: round(step_other_ms, 4)},
            "pair_overhead": run.pair_overhead, **single,
            "ring_steps": ring,
        }
    plan.close()

    if args.calibrate_copy:
        n = args.calibrate_copy * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        result["copy_calibration_bytes"] = 4 * n

    if not args.no_extras:
        del q, k, v, out, run
        torch.cuda.empty_cache()
        if not args.no_workloads:
            # the other block-sparse workloads: the causal one in the other layout, the video and
            # the skewed workload (LPT against round-robin order, with measured per-CU balance)
            others = {}
            if args.workload == "causal":
                other_layout = "striped" if args.layout == "contiguous" else "contiguous"
                others[f"causal_{other_layout}"] = workload_summary(bd, W, torch, dev, 3, other_layout)
            others["video"] = workload_summary(bd, W, torch, dev, 2)
            others["skewed"] = workload_summary(bd, W, torch, dev, 4, ring=True)
            result["workloads"] = others
        if not args.no_topk:
            result["topk_path"] = topk_path(bd, W, torch, dev)

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(w, min(args.cpu_heads, w.H))
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
