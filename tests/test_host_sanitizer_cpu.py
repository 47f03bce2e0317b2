"""The library's host code (validation, plan object, host LPT planner) built for the CPU under
AddressSanitizer and UndefinedBehaviorSanitizer (sparse_mask_load_amd/build_host_check.py), with
the host-side checks of test_abi_cpu.py run against that build in a child process that has the
sanitizer runtime preloaded.  Any sanitizer report fails the test."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_host_entry_points_under_address_and_undefined_behaviour_sanitizers():
    from sparse_mask_load_amd import build_host_check as HC

    lib = HC.build()
    syms = subprocess.run(["nm", "-D", lib], capture_output=True, text=True).stdout
    assert "__asan_" in syms and "__ubsan_" in syms  # the build is instrumented
    env = dict(os.environ)
    # the sanitizer runtime must come first among the preloaded libraries
    env["LD_PRELOAD"] = ":".join(p for p in (HC.runtime_preload(), os.environ.get("LD_PRELOAD", "")) if p)
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    r = subprocess.run([sys.executable, os.path.join(ROOT, "tests", "sanitized_host_run.py"), lib], env=env,
                       capture_output=True, text=True, timeout=900)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "SANITIZED HOST CHECKS OK" in r.stdout
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
