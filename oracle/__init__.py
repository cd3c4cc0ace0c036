"""Oracle for the tree-structured gated delta rule — TEST INFRASTRUCTURE ONLY.

Only the tests, ``__graft_entry__.smoke()`` and the bench's ``cpu_baseline``
leg may import this package. The product (``tree_forked_gated_amd``) never
does, and shares no code with it.

Contents:

* ``gdn_oracle.c`` — the per-token parent walk (TreeWY, "Speculative
  Verification for Gated DeltaNet Hybrids", section 1 Eq. 1 and section 3
  "Key rewrite"), built twice: fp64 (the parity reference) and fp32 (the
  "plain fp32 CPU implementation" that the bench times beside the GPU).
* ``closed_form.py`` — TreeWY Eq. 2 (one triangular system for all
  pseudo-values of a tree) and Eq. 3 (state of any node rebuilt from the
  pseudo-values), dense fp64, for tiny trees. It checks the walk.
* ``plan.py`` — the metadata the GPU builds (sequence, depth, segments,
  chunks, dependency levels, fork slots, ancestor masks), written from the
  definitions with plain loops.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gdn_oracle.c")
_LIBS = {"f64": os.path.join(_HERE, "liboracle_f64.so"), "f32": os.path.join(_HERE, "liboracle_f32.so")}
_loaded = {}

ERRORS = {0: "ok", -1: "bad arguments", -2: "bad parent", -3: "bad seq_start", -4: "bad path", -5: "no memory"}


def build(force: bool = True) -> None:
    """Compile the C oracle with gcc (fp64 and fp32 builds)."""
    for prec, lib in _LIBS.items():
        if not force and os.path.exists(lib) and os.path.getmtime(lib) >= os.path.getmtime(_SRC):
            continue
        cmd = ["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared", "-pthread", "-std=c99",
               "-Wall", "-o", lib + ".tmp", _SRC, "-lm"]
        if prec == "f32":
            cmd.insert(1, "-DORACLE_F32")
        subprocess.run(cmd, check=True)
        os.replace(lib + ".tmp", lib)


def _lib(prec: str) -> ctypes.CDLL:
    if prec not in _loaded:
        if not os.path.exists(_LIBS[prec]) or os.path.getmtime(_LIBS[prec]) < os.path.getmtime(_SRC):
            build(force=False)
        lib = ctypes.CDLL(_LIBS[prec])
        lib.oracle_forward.restype = ctypes.c_int
        lib.oracle_commit.restype = ctypes.c_int
        assert lib.oracle_real_size() == (8 if prec == "f64" else 4)
        _loaded[prec] = lib
    return _loaded[prec]


def _p(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def default_threads() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return max(1, os.cpu_count() or 1)


def forward(wl, precision: str = "f64", n_threads: Optional[int] = None, keep_pseudo: bool = True,
            state_rows: Optional[np.ndarray] = None, init_state="workload"):
    """Run the per-token walk over a workload.

    Returns a dict with ``out`` [T,H,Dv], ``pseudo_v`` [T,H,Dv] (when asked)
    and ``state`` [n_state,H,Dv,Dk] for ``state_rows`` (default: the
    workload's state rows), all in the oracle's precision.
    """
    dt = np.float64 if precision == "f64" else np.float32
    lib = _lib(precision)
    T, H, Dk, Dv, n_seq = wl.T, wl.H, wl.Dk, wl.Dv, wl.n_seq
    c = lambda a: np.ascontiguousarray(a, dtype=dt)
    q, k, v, g, b = c(wl.q), c(wl.k), c(wl.v), c(wl.log_gate), c(wl.beta)
    init = c(wl.init_state) if isinstance(init_state, str) else (None if init_state is None else c(init_state))
    rows = np.ascontiguousarray(wl.state_rows if state_rows is None else state_rows, dtype=np.int32)
    out = np.zeros((T, H, Dv), dtype=dt)
    pv = np.zeros((T, H, Dv), dtype=dt) if keep_pseudo else None
    st = np.zeros((rows.shape[0], H, Dv, Dk), dtype=dt)
    parent = np.ascontiguousarray(wl.parent, dtype=np.int32)
    seq = np.ascontiguousarray(wl.seq_start, dtype=np.int32)
    rc = lib.oracle_forward(ctypes.c_int64(T), H, Dk, Dv, n_seq, _p(seq), _p(parent), _p(q), _p(k), _p(v),
                            _p(g), _p(b), _p(init), _p(out), _p(pv), ctypes.c_int32(rows.shape[0]), _p(rows),
                            _p(st), n_threads or default_threads())
    if rc != 0:
        raise ValueError(f"oracle_forward: {ERRORS.get(rc, rc)}")
    return {"out": out, "pseudo_v": pv, "state": st}


def commit(wl, precision: str = "f64", n_threads: Optional[int] = None, path_ptr=None, path_nodes=None,
           path_seq=None):
    """Replay the accepted paths from the initial states (Eq. 3's result)."""
    dt = np.float64 if precision == "f64" else np.float32
    lib = _lib(precision)
    c = lambda a: np.ascontiguousarray(a, dtype=dt)
    pp = np.ascontiguousarray(wl.path_ptr if path_ptr is None else path_ptr, dtype=np.int32)
    pn = np.ascontiguousarray(wl.path_nodes if path_nodes is None else path_nodes, dtype=np.int32)
    ps = np.ascontiguousarray(wl.path_seq if path_seq is None else path_seq, dtype=np.int32)
    n_path = pp.shape[0] - 1
    out = np.zeros((n_path, wl.H, wl.Dv, wl.Dk), dtype=dt)
    rc = lib.oracle_commit(ctypes.c_int64(wl.T), wl.H, wl.Dk, wl.Dv, wl.n_seq,
                           _p(np.ascontiguousarray(wl.seq_start, dtype=np.int32)),
                           _p(np.ascontiguousarray(wl.parent, dtype=np.int32)), _p(c(wl.k)), _p(c(wl.v)),
                           _p(c(wl.log_gate)), _p(c(wl.beta)), _p(c(wl.init_state)), ctypes.c_int32(n_path),
                           _p(pp), _p(pn if pn.size else np.zeros(1, np.int32)), _p(ps), _p(out),
                           n_threads or default_threads())
    if rc != 0:
        raise ValueError(f"oracle_commit: {ERRORS.get(rc, rc)}")
    return out
