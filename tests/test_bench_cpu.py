"""bench.py's command-line contract that needs no GPU: one GPU only."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300)
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr)


def _bench():
    sys.path.insert(0, ROOT)
    import bench
    return bench


def test_counter_traffic_is_used_only_for_the_profiled_kernel_source(monkeypatch):
    bench = _bench()
    text = open(os.path.join(ROOT, "profiles", "attn_bf16_causal_hbm_counters.md")).read()
    profiled = text.split("kernel source hash: `")[1].split("`")[0]
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: profiled)
    traffic = bench.read_counter_traffic("causal")
    assert traffic is not None and traffic > 2.68e8  # at least Q, K, V read and O written once
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: "0" * 16)
    assert bench.read_counter_traffic("causal") is None
    assert bench.read_counter_traffic("no_such_workload") is None


def test_per_cu_balance_groups_items_by_hardware_cu():
    import numpy as np
    bench = _bench()
    # two XCCs; HW_ID bits 8-15 name the compute unit within one; bins in the upper half of word 3
    cu = lambda xcc, cu_id: (xcc << 32) | (cu_id << 8)
    rows = [  # start, end, hw location, bin << 32 | item
        (0, 10, cu(0, 1), (0 << 32) | 0),
        (10, 30, cu(0, 1), (0 << 32) | 1),   # CU (0, 1): 30
        (0, 20, cu(1, 1), (1 << 32) | 2),    # CU (1, 1): 20, same CU id on another XCC
        (0, 10, cu(0, 2), (2 << 32) | 3),    # CU (0, 2): 10
    ]
    out = bench.per_cu_balance(np.array(rows, dtype=np.int64))
    assert out["cus_used"] == 3
    assert abs(out["measured_cu_max_over_mean"] - 30 / 20) < 1e-12
    assert abs(out["measured_bin_max_over_mean"] - 30 / 20) < 1e-12
