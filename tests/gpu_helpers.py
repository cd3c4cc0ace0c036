"""Helpers of the GPU tests: move a workload to the device, run the library,
compare with the oracle. Nothing here computes any part of the recurrence."""
import json
import os
import sys
import time

import numpy as np
import torch

import oracle
from tree_forked_gated_amd import workloads as W


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def tdtype(wl):
    return torch.bfloat16 if wl.dtype == "bf16" else torch.float32


def to_device(wl, device="cuda"):
    dt = tdtype(wl)
    f = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device=device).to(dt).contiguous()
    return {
        "q": f(wl.q), "k": f(wl.k), "v": f(wl.v), "log_gate": f(wl.log_gate), "beta": f(wl.beta),
        "parent_idx": torch.from_numpy(wl.parent.astype(np.int32)).to(device),
        "seq_start": torch.from_numpy(wl.seq_start.astype(np.int32)).to(device),
        "init_state": torch.from_numpy(np.ascontiguousarray(wl.init_state, dtype=np.float32)).to(device),
    }


def run_forward(wl, keep_pseudo=None, state_rows=None, out_rows="workload", dv_tile=0, check=True, **kw):
    from tree_forked_gated_amd import binding as B
    d = to_device(wl)
    rows = wl.state_rows if state_rows is None else state_rows
    orows = wl.out_rows if isinstance(out_rows, str) else out_rows
    if "max_forks" not in kw:  # the exact capacities, from the structure held on the host
        kw.update(B.capacities(wl.parent, wl.seq_start))
    res = B.forward(d["q"], d["k"], d["v"], d["log_gate"], d["beta"], d["parent_idx"], d["seq_start"],
                    d["init_state"], out_rows=orows, state_rows=rows,
                    keep_pseudo=wl.keep_pseudo if keep_pseudo is None else keep_pseudo, dv_tile=dv_tile,
                    check=check, **kw)
    torch.cuda.synchronize()
    return res, d


def rel_l2(gpu, ref):
    g = np.asarray(gpu, dtype=np.float64)
    r = np.asarray(ref, dtype=np.float64)
    den = np.linalg.norm(r.ravel())
    return float(np.linalg.norm((g - r).ravel()) / (den if den > 0 else 1.0))


def tol(wl):
    return 1e-2 if wl.dtype == "bf16" else 1e-4


def f64(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def oracle_ref(wl, state_rows=None, keep_pseudo=True):
    return oracle.forward(wl, "f64", keep_pseudo=keep_pseudo, state_rows=state_rows)


def margin_log_path():
    """Where the parity margins go: $GDN_PARITY_LOG, else gpurun_out/ at the
    repository root (kept out of the repository's history)."""
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    return os.environ.get("GDN_PARITY_LOG", os.path.join(root, "gpurun_out", "parity_margins.jsonl"))


def record_margin(case, **values):
    """Append one JSON line with a case's error figures (relative L2 per
    tensor, worst row) so that the margins to the tolerances are kept."""
    path = margin_log_path()
    os.makedirs(os.path.dirname(path), exist_ok=True)
    rec = {"case": case, "time": round(time.time(), 1)}
    rec.update({k: (float(f"{v:.4e}") if isinstance(v, float) else v) for k, v in values.items()})
    with open(path, "a") as f:
        f.write(json.dumps(rec) + "\n")
