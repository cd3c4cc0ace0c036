"""The oracle and the HIP path share no code, and the product path has no CPU
fallback: the library and the binding never import, include or call anything
under oracle/, the oracle imports nothing of the package (tests hand it the
seeded workloads), and the binding refuses to load without the built HIP
library."""
import os
import re
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "tree_forked_gated_amd")


def _files(top, exts):
    for d, _, names in os.walk(top):
        if "_build" in d or "__pycache__" in d:
            continue
        for n in names:
            if n.endswith(exts):
                yield os.path.join(d, n)


def test_product_never_reaches_the_oracle():
    bad = []
    for p in _files(PKG, (".py",)):
        for ln, line in enumerate(open(p), 1):
            if re.match(r"\s*(import\s+oracle\b|from\s+oracle\b)", line) or "liboracle" in line:
                bad.append(f"{os.path.relpath(p, ROOT)}:{ln}")
    for p in list(_files(PKG, (".hip", ".h", ".cpp"))) + list(_files(os.path.join(ROOT, "include"), (".h",))):
        for ln, line in enumerate(open(p), 1):
            if re.match(r"\s*#\s*include\s*[<\"].*oracle", line):
                bad.append(f"{os.path.relpath(p, ROOT)}:{ln}")
    assert not bad, bad


def test_oracle_imports_nothing_of_the_package():
    bad = []
    for p in _files(os.path.join(ROOT, "oracle"), (".py", ".c")):
        for ln, line in enumerate(open(p), 1):
            if re.match(r"\s*(import|from)\s+tree_forked_gated_amd\b", line) or re.match(r"\s*#\s*include\s*\"", line):
                bad.append(f"{os.path.relpath(p, ROOT)}:{ln}")
    assert not bad, bad


def test_binding_fails_loudly_without_the_hip_library(tmp_path):
    env = dict(os.environ, GDN_TREE_LIB=str(tmp_path / "missing.so"), PYTHONPATH=ROOT)
    r = subprocess.run([sys.executable, "-c", "import tree_forked_gated_amd.binding"], env=env, cwd=str(tmp_path),
                       capture_output=True, text=True, timeout=300)
    assert r.returncode != 0
    assert "missing.so" in r.stderr
