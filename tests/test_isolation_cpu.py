"""The oracle and the HIP path share no code, and the product path has no fallback."""
import os
import re
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(code: str) -> subprocess.CompletedProcess:
    return subprocess.run([sys.executable, "-c", code], cwd=ROOT, capture_output=True, text=True, timeout=300)


def test_package_does_not_import_the_oracle():
    r = _run("import sys; import sparse_mask_load_amd, sparse_mask_load_amd.binding, sparse_mask_load_amd.workloads, "
             "sparse_mask_load_amd.build; print(sorted(m for m in sys.modules if m == 'oracle' or m.startswith('oracle.')))")
    assert r.returncode == 0, r.stderr
    assert r.stdout.strip() == "[]"


def test_oracle_does_not_import_the_package():
    r = _run("import sys; import oracle.attention, oracle.plan, oracle.topk; "
             "print(sorted(m for m in sys.modules if m.startswith('sparse_mask_load_amd')))")
    assert r.returncode == 0, r.stderr
    assert r.stdout.strip() == "[]"


def test_no_source_of_one_side_names_the_other():
    pat_oracle = re.compile(r"^\s*(from|import)\s+oracle\b", re.M)
    for d in ("sparse_mask_load_amd", "include"):
        for dirpath, _, files in os.walk(os.path.join(ROOT, d)):
            for f in files:
                if f.endswith((".py", ".hip", ".cpp", ".h")):
                    text = open(os.path.join(dirpath, f), errors="ignore").read()
                    assert not pat_oracle.search(text), f"{f} imports the oracle"
                    assert "oracle/" not in text, f"{f} names the oracle's files"
    pat_pkg = re.compile(r"^\s*(from|import)\s+sparse_mask_load_amd\b", re.M)
    for f in os.listdir(os.path.join(ROOT, "oracle")):
        if f.endswith(".py"):
            assert not pat_pkg.search(open(os.path.join(ROOT, "oracle", f)).read()), f"oracle/{f} imports the package"


def test_binding_raises_without_the_library():
    r = _run("from sparse_mask_load_amd import binding as b\n"
             "b.LIB_PATH = '/nonexistent/libsparse_attn.so'\n"
             "try:\n    b.lib()\nexcept RuntimeError as e:\n    print('raised', 'not built' in str(e))\n")
    assert r.returncode == 0, r.stderr
    assert r.stdout.strip() == "raised True"
