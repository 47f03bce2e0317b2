"""Host-only build of the C ABI under AddressSanitizer and UndefinedBehaviorSanitizer.

Compiles the host sources (validation, plan object, host LPT planner: api.cpp, lpt.cpp) with the
kernel launchers replaced by stubs (host_check_stubs.cpp), as plain C++ for the CPU, into
``_build/host_check/libsparse_attn_host_check.so``.  The host entry points
(``sparse_attn_assign_host``, ``sparse_attn_assign_host_grouped``, argument checks) can then run
under the sanitizers on a machine without a GPU.  A process that loads the library needs the
sanitizer runtime preloaded (see ``runtime_preload()``).

Usage: ``python -m sparse_mask_load_amd.build_host_check``.
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OUT_DIR = os.path.join(ROOT, "_build", "host_check")
LIB = os.path.join(OUT_DIR, "libsparse_attn_host_check.so")
ROCM = "/opt/rocm"
CXX = os.path.join(ROCM, "llvm", "bin", "clang++")  # a host C++ compiler that knows __bf16
SOURCES = ["api.cpp", "lpt.cpp", "host_check_stubs.cpp"]
SANITIZE = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-shared-libasan"]


def runtime_preload() -> str:
    """Path of the AddressSanitizer runtime that must be preloaded into a process using LIB."""
    hits = sorted(glob.glob(os.path.join(ROCM, "llvm", "lib", "clang", "*", "lib", "linux",
                                         "libclang_rt.asan-x86_64.so")))
    if not hits:
        raise RuntimeError("AddressSanitizer runtime of the ROCm clang not found")
    return hits[-1]


def build() -> str:
    os.makedirs(OUT_DIR, exist_ok=True)
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    cmd = [CXX, "-x", "c++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fPIC", "-shared",
           "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           "-I", os.path.join(ROCM, "include"), *SANITIZE, *srcs,
           "-L", os.path.join(ROCM, "lib"), "-lamdhip64", "-o", LIB]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"host check build failed:\n{' '.join(cmd)}\n{res.stdout}{res.stderr}")
    return LIB


if __name__ == "__main__":
    print(build())
    print(runtime_preload())
