"""Runs the host-side checks of tests/test_abi_cpu.py (host LPT planner bit-exact against the
oracle, argument validation) against the sanitizer build of the library's host code.  Started by
tests/test_host_sanitizer_cpu.py in a process that has the sanitizer runtime preloaded; the path
of the library is the first argument."""
import ctypes
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

from sparse_mask_load_amd import binding as bd  # noqa: E402

handle = ctypes.CDLL(sys.argv[1])
for name, (res, args) in bd._SIGNATURES.items():
    if hasattr(handle, name):  # the host build has no allocation-free (device-only) entry point
        fn = getattr(handle, name)
        fn.restype = res
        fn.argtypes = args
bd._lib = handle  # the binding's calls now go to the sanitizer build

from tests import test_abi_cpu as T  # noqa: E402

T.test_status_strings()
for order in ("lpt", "naive"):
    T.test_host_assign_bit_exact_random(order)
T.test_host_assign_bit_exact_large_loads()
T.test_host_assign_page_example()
for cfg, m in ((2, 512), (3, 256), (4, 256)):
    T.test_host_assign_bit_exact_on_workload_rows(cfg, m)
T.test_host_assign_errors()
T.test_host_grouped_assign_bit_exact_random()
for cfg, m in ((3, 256), (4, 256)):
    T.test_host_grouped_assign_on_workload_rows(cfg, m)
for kw, status in T.BAD_PROBLEMS:
    T.test_plan_rejects_bad_problems_before_touching_the_gpu(kw, status)
T.test_problem_fields_are_the_declared_ones()
T.test_token_causal_only_for_block_plans()
T.test_q_pairs_only_for_block_plans()
T.test_hip_errors_surface_as_sa_err_hip()
for order in (bd.SA_ORDER_LPT_DEVICE, bd.SA_ORDER_LPT_DYNAMIC):
    T.test_device_order_limits_checked_before_the_gpu(order)
T.test_fwd_and_merge_argument_errors()
print("SANITIZED HOST CHECKS OK", flush=True)
