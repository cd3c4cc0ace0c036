"""Per-stage cycle counts of the walk, from its stage stamps (a measurement build).

`build.build(stamps=True)` compiles libgdn_tree_stamps.so: the same sources with
the walk's stage stamps compiled in (-DGDN_WALK_STAMPS). Lane 0 of every wave of
the first eight workgroups of the first level launch records s_memtime at each
stage boundary of its first 128 chunks. This script runs one planned forward of
a workload through that library and prints, for the waves of the first two
workgroups, the median cycles per stage over their chunks (the first two and
the last two dropped). Each stamp costs about 100 cycles. With two 16-column
blocks per state wave (d_v tiles of 64) the kernel has no scheduling barriers
between stages, so there only the per-chunk total is reliable.

    python -m tree_forked_gated_amd.stage_stamps --build-only     # on the host
    python -m tree_forked_gated_amd.stage_stamps --workload chains  # on a GPU
"""
from __future__ import annotations

import argparse
import ctypes
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
STAMPS_LIB = os.path.join(HERE, "libgdn_tree_stamps.so")
WG, WAVES, ITS, PTS = 8, 4, 128, 10  # the stamp array's shape (walk_pipe.hip)

STATE_STAGES = ["K S_e^T", "S_e Q^T", "R", "substitution", "P Vt + outputs", "pseudo-values", "exit update",
                "next descriptor", "entry-state loads", "barrier wait"]
HELPER_STAGES = ["copies issued", "products", "wait for copies", "token tables | item feed", "barrier wait"]


def _medians(S, wg, w, helper):
    its = [i for i in range(ITS) if S[wg, w, i, 0] != 0]
    rows = []
    for i in its:
        r = S[wg, w, i]
        nxt = S[wg, w, i + 1, 0] if i + 1 < ITS else 0
        if not nxt:
            continue
        if helper:
            rows.append([r[1] - r[0], r[2] - r[1], r[3] - r[2], r[4] - r[3], nxt - r[4]])
        else:
            rows.append([r[k + 1] - r[k] for k in range(9)] + [nxt - r[9]])
    if not rows:
        return None, 0
    a = np.array(rows[2:-2] if len(rows) > 6 else rows, np.float64)
    per_chunk = float(np.median(np.diff([S[wg, w, i, 0] for i in its])))
    return np.median(a, axis=0), per_chunk


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--workload", default="chains")
    ap.add_argument("--build-only", action="store_true")
    ap.add_argument("--no-build", action="store_true")
    args = ap.parse_args()
    if not args.no_build:
        sys.path.insert(0, HERE)
        import build as _build
        print("built", _build.build(stamps=True), flush=True)
        if args.build_only:
            return
    os.environ["GDN_TREE_LIB"] = STAMPS_LIB
    import torch
    from tree_forked_gated_amd import binding as B
    from tree_forked_gated_amd import workloads as W
    assert B.LIB_PATH == STAMPS_LIB, B.LIB_PATH
    B.lib.gdn_walk_stamps.argtypes = [ctypes.c_void_p, ctypes.c_int]
    wl = W.get(args.workload)
    print(f"workload {wl.name}: T={wl.T} H={wl.H}", flush=True)
    dev = torch.device("cuda:0")
    dt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32

    def f(x):
        return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(dev).to(dt).contiguous()

    q, k, v, g, b = f(wl.q), f(wl.k), f(wl.v), f(wl.log_gate), f(wl.beta)
    init = torch.from_numpy(np.ascontiguousarray(wl.init_state, np.float32)).to(dev)
    parent = torch.from_numpy(wl.parent.astype(np.int32)).to(dev)
    ss = torch.from_numpy(wl.seq_start.astype(np.int32)).to(dev)
    out_rows = None if wl.out_rows is None else wl.out_rows
    cap = B.capacities(wl.parent, wl.seq_start)
    kw = dict(out_rows=out_rows, state_rows=wl.state_rows, keep_pseudo=wl.keep_pseudo,
              max_forks=cap["max_forks"], max_levels=cap["max_levels"])
    res = B.forward(q, k, v, g, b, parent, ss, init, **kw)
    torch.cuda.synchronize()
    B.lib.gdn_walk_stamps(None, 1)
    torch.cuda.synchronize()
    B.forward(q, k, v, g, b, parent, ss, init, workspace=res.workspace, out=res.out, state_out=res.state,
              pseudo_v=res.pseudo_v, planned=True, **kw)
    torch.cuda.synchronize()
    buf = np.zeros(WG * WAVES * ITS * PTS, np.uint64)
    rc = B.lib.gdn_walk_stamps(buf.ctypes.data_as(ctypes.c_void_p), 0)
    if rc != 0:
        raise RuntimeError(f"gdn_walk_stamps: hip error {rc}")
    S = buf.reshape(WG, WAVES, ITS, PTS).astype(np.int64)
    for wg in range(2):
        for w in range(WAVES):
            if not S[wg, w, :, 0].any():
                continue
            # helper waves stamp 5 points; state waves stamp all 10
            helper = not S[wg, w, :, 9].any()
            med, per = _medians(S, wg, w, helper)
            if med is None:
                continue
            names = HELPER_STAGES if helper else STATE_STAGES
            cells = ", ".join(f"{nm} {m:.0f}" for nm, m in zip(names, med))
            print(f"workgroup {wg} wave {w} ({'helper' if helper else 'state'}): {per:.0f} cycles per chunk; {cells}",
                  flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
