"""Benchmark of the block-sparse attention hot path on one MI355X.

One step = one pass of the whole path over one batch of the causal long-sequence
workload (B1 H16 S16384 d128, block 128, lower-triangular block mask, KV in 4 contiguous
chunks, one bin per compute unit):

  1. sparse_attn_plan: GPU popcount of the mask and the work lists, by default with the
     device planner (round-based LPT made on the GPU; --order lpt_xcd / lpt / naive plan
     on the host instead).  The mask is a runtime input, so every step re-plans, on a
     side stream; the forward call waits for the plan's event;
  2. sparse_attn_fwd in partial mode over chunks [0, 4): one (O, m, l) partial per chunk;
  3. chunk_merge: online-softmax merge of the 4 partials into O (bf16).

value = live-block FLOP per step (4 * 128^3 per live tile) / measured step time.

The untimed extras also run the token top-k path on its own workload (B1 H16 n32768 d128,
rank-32 indexer, top-k 512, causal): the TOPK plan (projections + importance + per-query
top-k) and the gather attention over the selected keys, reported as times and rates.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--mode merged|fused]
       [--workload causal|video|skewed|tiny] [--no-cpu-baseline] [--calibrate-copy MiB]
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
KERNEL_NAME = "attn_bf16_kernel"
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


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", choices=sorted(WORKLOADS), default="causal")
    ap.add_argument("--mode", choices=["merged", "fused"], default="merged",
                    help="merged: partial chunks + chunk_merge (default); fused: chunks folded in-kernel")
    ap.add_argument("--order", choices=["lpt_xcd", "lpt", "naive", "lpt_device"], default="lpt_device",
                    help="work order: two-level LPT (heads to XCDs, then Q-blocks), one-level LPT, round-robin, "
                         "round-based LPT made on the GPU")
    ap.add_argument("--bins", type=int, default=0, help="persistent workgroups (0: one per resident slot)")
    ap.add_argument("--cpu-heads", type=int, default=12, help="heads of the oracle's timed sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true", help="skip the untimed breakdown runs")
    ap.add_argument("--no-topk", action="store_true", help="skip the token top-k path measurement")
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

    w = W.make(WORKLOADS[args.workload])
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    q, k, v = (torch.from_numpy(x).to(dev, dt) for x in (w.q, w.k, w.v))
    mask = torch.from_numpy(w.mask).to(dev)
    B, H, S, D = q.shape
    C = w.n_chunks
    prob = bd.make_problem(q, w.block, C, w.layout)
    o_part = torch.empty((C, B, H, S, D), dtype=torch.float32, device=dev)
    m_part = torch.empty((C, B, H, S), dtype=torch.float32, device=dev)
    l_part = torch.empty((C, B, H, S), dtype=torch.float32, device=dev)
    out = torch.empty_like(q)
    rows = B * H * S
    stream = torch.cuda.current_stream()
    # the plan of a step is built on a side stream: its host part (counts, LPT, uploads) then
    # overlaps the previous step's attention on the main stream, and the forward call waits
    # for the plan's uploads by itself
    plan_stream = torch.cuda.Stream()
    fwd_events = []

    def step(record: bool):
        plan = bd.sparse_attn_plan(prob, "block", mask=mask, order=args.order, num_bins=args.bins, stream=plan_stream)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        if args.mode == "merged":
            bd.sparse_attn_fwd(plan, q, k, v, 0, C, o_part=o_part, m_part=m_part, l_part=l_part)
            e1.record(stream)
            bd.chunk_merge([o_part[c] for c in range(C)], [m_part[c] for c in range(C)],
                           [l_part[c] for c in range(C)], rows, D, out, w.dtype)
        else:
            bd.sparse_attn_fwd(plan, q, k, v, 0, C, o=out)
            e1.record(stream)
        if record:
            fwd_events.append((e0, e1))
        return plan

    for _ in range(args.warmup):
        step(False).close()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    plans = []  # destroyed after the timed region (destroying a plan synchronises the device)
    for _ in range(args.steps):
        plans.append(step(True))
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for p in plans:
        p.close()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    kernel_ms = float(np.mean([a.elapsed_time(b) for a, b in fwd_events]))

    plan = bd.sparse_attn_plan(prob, "block", mask=mask, order=args.order, num_bins=args.bins)
    info = bd.sparse_attn_plan_info(plan)
    flop = 4.0 * w.block * w.block * D * info["total_live"]
    value = flop / (ms_per_step * 1e-3) / 1e12
    achieved = flop / (kernel_ms * 1e-3) / 1e12
    bin_load = bd.sparse_attn_plan_copy(plan, bd.SA_PLAN_BIN_LOAD, info["num_bins"])

    result = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": f"{w.name} block-sparse MHA B{B} H{H} S{S} d{D} block {w.block}, "
                               f"{C} {w.layout} KV chunks {'merged by chunk_merge' if args.mode == 'merged' else 'folded in-kernel'}, "
                               f"{ {'lpt_xcd': 'two-level LPT (heads to XCDs, then Q-blocks)', 'lpt': 'LPT', 'naive': 'round-robin', 'lpt_device': 'round-based LPT made on the GPU'}[args.order]} over {info['num_bins']} bins",
                   "B": B, "H": H, "S": S, "D": D, "block": w.block, "n_chunks": C, "layout": w.layout,
                   "mask": {"tiny": "Bernoulli(0.5)+diag", "video": "frame band / Bernoulli",
                            "causal": "block lower-triangular", "skewed": "Zipf(1.2) rows"}[args.workload],
                   "live_tiles": info["total_live"], "mode": args.mode, "order": args.order},
        "pct_bf16_peak_step": round(100.0 * value / PEAK_BF16_TFLOPS, 2),
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": read_counter_traffic(args.workload),
                     "kernel": KERNEL_NAME, "kernel_ms": round(kernel_ms, 4),
                     "kernel_source_hash": kernel_source_hash()},
        "per_cu_work": {"planned_bin_max_over_mean": round(float(bin_load.max() / bin_load.mean()), 4),
                        "planned_makespan_tiles": info["makespan"], "lower_bound_tiles": info["lower_bound"]},
    }

    if not args.no_extras:
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        # per-CU busy time from the in-kernel trace (one untimed launch)
        trace = torch.zeros((info["n_items"], 4), dtype=torch.int64, device=dev)
        bd.sparse_attn_fwd(plan, q, k, v, 0, C, o=out, trace=trace)
        torch.cuda.synchronize()
        result["per_cu_work"].update(per_cu_balance(trace.cpu().numpy()))
        # fused (in-kernel chunk fold) forward and the merge alone; every timed loop below
        # starts after one untimed launch of the same call (clock ramp after host work, an
        # asynchronous plan's completion)
        reps = 10
        bd.sparse_attn_fwd(plan, q, k, v, 0, C, o=out)
        e0.record(stream)
        for _ in range(reps):
            bd.sparse_attn_fwd(plan, q, k, v, 0, C, o=out)
        e1.record(stream)
        torch.cuda.synchronize()
        fused_ms = e0.elapsed_time(e1) / reps
        bd.chunk_merge([o_part[c] for c in range(C)], [m_part[c] for c in range(C)], [l_part[c] for c in range(C)],
                       rows, D, out, w.dtype)
        e0.record(stream)
        for _ in range(reps):
            bd.chunk_merge([o_part[c] for c in range(C)], [m_part[c] for c in range(C)], [l_part[c] for c in range(C)],
                           rows, D, out, w.dtype)
        e1.record(stream)
        torch.cuda.synchronize()
        merge_ms = e0.elapsed_time(e1) / reps
        merge_bytes = rows * (C * (D * 4 + 8) + D * (2 if w.dtype == "bf16" else 4))
        t_plan = time.perf_counter()
        for _ in range(reps):  # host planner (waits for the counts, LPT on the host)
            bd.sparse_attn_plan(prob, "block", mask=mask, order="lpt_xcd").close()
        plan_host_ms = (time.perf_counter() - t_plan) * 1e3 / reps
        # device planner: host cost of the call (it returns without waiting) and its GPU time
        t_plan = time.perf_counter()
        dplans = [bd.sparse_attn_plan(prob, "block", mask=mask, order="lpt_device") for _ in range(reps)]
        plan_device_call_ms = (time.perf_counter() - t_plan) * 1e3 / reps
        torch.cuda.synchronize()
        for p_d in dplans:
            p_d.close()
        gpu_ms = []
        for _ in range(reps):  # device-side latency: mask copy, popcount and the planning kernel
            e0.record(stream)
            p_d = bd.sparse_attn_plan(prob, "block", mask=mask, order="lpt_device", stream=stream)
            e1.record(stream)
            torch.cuda.synchronize()
            gpu_ms.append(e0.elapsed_time(e1))
            p_d.close()
        plan_device_gpu_ms = float(np.median(gpu_ms))
        # whole steps with the other planner (same loop as the timed one)
        order_main = args.order
        other_order = "lpt_xcd" if order_main == "lpt_device" else "lpt_device"
        args.order = other_order
        for _ in range(2):
            step(False).close()
        torch.cuda.synchronize()
        t_dev = time.perf_counter()
        dplans = [step(False) for _ in range(args.steps)]
        torch.cuda.synchronize()
        step_other_ms = (time.perf_counter() - t_dev) * 1e3 / args.steps
        for p_d in dplans:
            p_d.close()
        args.order = order_main
        alt_ms = {}
        # persistent orders over one bin per resident workgroup, then one item per workgroup
        # (a plain grid that the hardware dispatches as compute units free up), in id order
        # and in LPT order
        n_items = info["n_items"]
        alts = [(o_, o_, 0) for o_ in ("naive", "lpt", "lpt_xcd", "lpt_device")]
        alts += [("grid_id_order", "naive", n_items), ("grid_lpt_order", "lpt", n_items)]
        for alt, alt_order, alt_bins in alts:
            p_alt = bd.sparse_attn_plan(prob, "block", mask=mask, order=alt_order, num_bins=alt_bins)
            bd.sparse_attn_fwd(p_alt, q, k, v, 0, C, o=out)
            e0.record(stream)
            for _ in range(reps):
                bd.sparse_attn_fwd(p_alt, q, k, v, 0, C, o=out)
            e1.record(stream)
            torch.cuda.synchronize()
            alt_ms[alt] = (e0.elapsed_time(e1) / reps, bd.sparse_attn_plan_info(p_alt))
            p_alt.close()
        # the same mask with token-level causality inside the live tiles
        p_tc = bd.sparse_attn_plan(bd.make_problem(q, w.block, C, w.layout, token_causal=True), "block",
                                   mask=mask, order=args.order)
        bd.sparse_attn_fwd(p_tc, q, k, v, 0, C, o=out)
        e0.record(stream)
        for _ in range(reps):
            bd.sparse_attn_fwd(p_tc, q, k, v, 0, C, o=out)
        e1.record(stream)
        torch.cuda.synchronize()
        tc_ms = e0.elapsed_time(e1) / reps
        p_tc.close()

        # the partial-mode forward with cold caches: a 512 MiB write first evicts the L2s and
        # the Infinity Cache (256 MiB), so Q, K and V come from HBM (median of 3)
        evict = torch.empty(128 << 20, dtype=torch.float32, device=dev)
        cold = []
        for _ in range(3):
            evict.fill_(1.0)
            e0.record(stream)
            bd.sparse_attn_fwd(plan, q, k, v, 0, C, o_part=o_part, m_part=m_part, l_part=l_part)
            e1.record(stream)
            torch.cuda.synchronize()
            cold.append(e0.elapsed_time(e1))
        del evict
        partial_cold_ms = float(np.median(cold))
        # measured per-CU balance of the round-robin order, beside the step's planner above
        p_naive = bd.sparse_attn_plan(prob, "block", mask=mask, order="naive")
        tr_naive = torch.zeros((info["n_items"], 4), dtype=torch.int64, device=dev)
        bd.sparse_attn_fwd(p_naive, q, k, v, 0, C, o=out, trace=tr_naive)
        torch.cuda.synchronize()
        naive_balance = per_cu_balance(tr_naive.cpu().numpy())
        p_naive.close()
        props = torch.cuda.get_device_properties(dev)
        result["device"] = {"name": props.name, "arch": getattr(props, "gcnArchName", None),
                            "compute_units": props.multi_processor_count, "peak_clock_mhz": peak_clock_mhz(dev.index or 0)}
        result["per_cu_work"]["naive_measured_cu_max_over_mean"] = naive_balance["measured_cu_max_over_mean"]
        result["breakdown"] = {
            "plan_host_ms": round(plan_host_ms, 4), "fwd_partial_ms": round(kernel_ms, 4),
            "fwd_partial_cold_ms": round(partial_cold_ms, 4),
            "fwd_fused_ms": round(fused_ms, 4), "fused_tflops": round(flop / fused_ms / 1e9, 2),
            "fused_pct_bf16_peak": round(100 * flop / fused_ms / 1e9 / PEAK_BF16_TFLOPS, 2),
            "merge_ms": round(merge_ms, 4), "merge_gbs": round(merge_bytes / merge_ms / 1e6, 1),
            "fwd_fused_ms_by_order": {o: round(t, 4) for o, (t, _) in alt_ms.items()},
            "makespan_tiles_by_order": {o: i["makespan"] for o, (_, i) in alt_ms.items()},
            "xcd_groups": alt_ms["lpt_xcd"][1]["groups"],
            "fwd_fused_token_causal_ms": round(tc_ms, 4),
            "plan_device_call_ms": round(plan_device_call_ms, 4), "plan_device_gpu_ms": round(plan_device_gpu_ms, 4),
            "ms_per_step_by_planner": {order_main: round(ms_per_step, 4), other_order: round(step_other_ms, 4)},
        }
    plan.close()

    if args.calibrate_copy:
        n = args.calibrate_copy * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        result["copy_calibration_bytes"] = 4 * n

    if not args.no_extras and not args.no_topk:
        del q, k, v, o_part, m_part, l_part, out
        torch.cuda.empty_cache()
        result["topk_path"] = topk_path(bd, W, torch, dev)

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(w, min(args.cpu_heads, w.H))
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
