"""The C oracle under AddressSanitizer and UndefinedBehaviorSanitizer (CPU).

The oracle's walk and commit are built again with -fsanitize=address,undefined
(no recovery) and run, through the same Python wrapper, on seeded streams of
chains, draft trees and nested forests in both precisions and on several
threads, and on malformed structures that it must refuse without reading out
of bounds. The run happens in a child process that preloads the sanitizer
runtime ahead of whatever is already preloaded; a planted heap overflow and a
planted out-of-range index, built and run the same way, must be caught (the
negative controls)."""
import os
import subprocess
import sys
import textwrap

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_oracle_under_address_and_undefined_sanitizers(tmp_path):
    asan = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    if not os.path.isabs(asan) or not os.path.exists(asan):
        pytest.skip("gcc has no AddressSanitizer runtime here")
    src = os.path.join(ROOT, "oracle", "gdn_oracle.c")
    libs = {}
    for prec in ("f64", "f32"):
        out = str(tmp_path / f"liboracle_{prec}.so")
        cmd = ["gcc", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
               "-fno-omit-frame-pointer", "-ffp-contract=off", "-fPIC", "-shared", "-pthread", "-std=c99", "-o", out,
               src, "-lm"]
        if prec == "f32":
            cmd.insert(1, "-DORACLE_F32")
        subprocess.run(cmd, check=True)
        libs[prec] = out
    script = textwrap.dedent(f"""
        import numpy as np
        import oracle
        from tree_forked_gated_amd import workloads as W
        oracle._LIBS.update({libs!r})
        runs = 0
        for seed in range(3):
            wl = W.random_small(seed + 70, n_seq=5, H=2, Dk=16, Dv=32, dtype="f32", max_len=150)
            leaves = W.leaves_of(wl.parent)
            ptr, nodes = [0], []
            for t in leaves[:6]:
                nodes += W.root_path(wl.parent, int(t))
                ptr.append(len(nodes))
            seqs = np.searchsorted(wl.seq_start, leaves[:6], side="right").astype(np.int32) - 1
            for prec in ("f64", "f32"):
                ref = oracle.forward(wl, prec, n_threads=3, keep_pseudo=True, state_rows=leaves)
                assert all(np.isfinite(v).all() for v in ref.values() if isinstance(v, np.ndarray))
                c = oracle.commit(wl, prec, n_threads=3, path_ptr=np.array(ptr, np.int32),
                                  path_nodes=np.array(nodes, np.int32), path_seq=seqs)
                assert np.isfinite(c).all()
                runs += 1
        wl = W.random_small(5, n_seq=3, H=1, Dk=16, Dv=16, dtype="f32", max_len=60)
        for t, p in [(5, 5), (7, 10**6), (9, -7)]:
            bad = wl.parent.copy()
            bad[t] = p
            wl2 = W.Workload("bad", "f32", bad, wl.seq_start, wl.q, wl.k, wl.v, wl.beta, wl.log_gate,
                             wl.init_state, None, np.zeros(0, np.int32))
            try:
                oracle.forward(wl2, "f64")
            except ValueError:
                runs += 1
        print("sanitized oracle ok", runs)
    """)
    env = dict(os.environ, PYTHONPATH=ROOT, ASAN_OPTIONS="detect_leaks=0",
               LD_PRELOAD=(asan + " " + os.environ.get("LD_PRELOAD", "")).strip())
    r = subprocess.run([sys.executable, "-c", script], env=env, capture_output=True, text=True, timeout=600,
                       cwd=str(tmp_path))
    assert r.returncode == 0, r.stderr[-4000:]
    assert "sanitized oracle ok 9" in r.stdout, r.stdout[-2000:]
    # negative controls: the same build and run catch a planted heap overflow
    # (AddressSanitizer) and a planted out-of-range array index (UndefinedBehaviorSanitizer)
    (tmp_path / "planted.c").write_text(
        "#include <stdlib.h>\n"
        "int heap_oob(int i) { int* a = malloc(4 * sizeof(int)); for (int j = 0; j < 4; ++j) a[j] = j;\n"
        "  int v = ((volatile int*)a)[i]; free(a); return v; }\n"
        "int index_oob(int i) { int a[4] = {1, 2, 3, 4}; return a[i]; }\n")
    for fn, flag, want in (("heap_oob", "address", "AddressSanitizer"), ("index_oob", "undefined", "runtime error")):
        lib = str(tmp_path / f"libplanted_{flag}.so")
        subprocess.run(["gcc", "-O1", "-g", f"-fsanitize={flag}", "-fno-sanitize-recover=all", "-fPIC", "-shared",
                        "-o", lib, str(tmp_path / "planted.c")], check=True)
        probe = f"import ctypes; print(ctypes.CDLL({lib!r}).{fn}(6))"
        r = subprocess.run([sys.executable, "-c", probe], env=env, capture_output=True, text=True, timeout=300)
        assert r.returncode != 0 and want in r.stderr, (fn, r.returncode, r.stderr[-2000:])
