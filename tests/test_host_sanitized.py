"""The library's host code under AddressSanitizer (CPU).

Every HIP source is compiled again with AddressSanitizer on its host part only
(-Xarch_host before each sanitizer flag; the GPU code is built as usual) and
linked into a library of its own. The CPU ABI tests (argument checks, sizes,
layouts, exported symbols) then run against that library in a child process
that preloads the compiler's sanitizer runtime ahead of whatever is already
preloaded. A planted heap overflow in host code, built and run the same way,
must be caught (the negative control)."""
import concurrent.futures as cf
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HOST_ASAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer"]


def _runtime(hipcc):
    llvm = os.path.join(os.path.dirname(os.path.dirname(os.path.realpath(hipcc))), "lib", "llvm")
    hits = sorted(glob.glob(os.path.join(llvm, "lib", "clang", "*", "lib", "linux", "libclang_rt.asan-x86_64.so")))
    return hits[-1] if hits else None


def _env(rt, lib=None):
    env = dict(os.environ, PYTHONPATH=ROOT, ASAN_OPTIONS="detect_leaks=0",
               LD_PRELOAD=(rt + " " + os.environ.get("LD_PRELOAD", "")).strip())
    if lib:
        env["GDN_TREE_LIB"] = lib
    return env


def test_host_code_under_address_sanitizer(tmp_path):
    from tree_forked_gated_amd import build as hipbuild
    hipcc = hipbuild.HIPCC
    rt = _runtime(hipcc) if os.path.exists(hipcc) else None
    if rt is None:
        pytest.skip("no hipcc or no AddressSanitizer runtime for it here")

    def one(src):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        cmd = [hipcc, *hipbuild.FLAGS, *hipbuild.FILE_FLAGS.get(os.path.basename(src), []), *HOST_ASAN, "-c", src,
               "-o", obj]
        subprocess.run(cmd, check=True, capture_output=True)
        return obj

    with cf.ThreadPoolExecutor(min(8, os.cpu_count() or 4)) as ex:
        objs = list(ex.map(one, hipbuild.sources()))
    lib = str(tmp_path / "libgdn_tree_host_asan.so")
    subprocess.run([hipcc, "-shared", "-fPIC", f"--offload-arch={hipbuild.ARCH}", "-Xarch_host", "-fsanitize=address",
                    "-Xarch_host", "-shared-libsan", *objs, "-o", lib], check=True, capture_output=True)
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_abi_cpu.py"), "-q",
                        "-p", "no:cacheprovider", "-m", "not gpu"], env=_env(rt, lib), capture_output=True, text=True,
                       timeout=600, cwd=str(tmp_path))
    assert r.returncode == 0, (r.stdout[-3000:], r.stderr[-3000:])
    assert "AddressSanitizer" not in r.stderr
    # negative control: a planted heap overflow in host code is caught
    src = tmp_path / "planted.hip"
    src.write_text('#include <cstdlib>\nextern "C" int heap_oob(int i) {\n  int* a = (int*)malloc(4 * sizeof(int));\n'
                   '  for (int j = 0; j < 4; ++j) a[j] = j;\n  int v = ((volatile int*)a)[i];\n  free(a);\n  return v;\n}\n')
    plib = str(tmp_path / "libplanted.so")
    subprocess.run([hipcc, "-O1", "-fPIC", "-shared", f"--offload-arch={hipbuild.ARCH}", *HOST_ASAN, "-Xarch_host",
                    "-shared-libsan", str(src), "-o", plib], check=True, capture_output=True)
    probe = f"import ctypes; print(ctypes.CDLL({plib!r}).heap_oob(6))"
    r = subprocess.run([sys.executable, "-c", probe], env=_env(rt), capture_output=True, text=True, timeout=300)
    assert r.returncode != 0 and "AddressSanitizer" in r.stderr, (r.returncode, r.stderr[-2000:])
