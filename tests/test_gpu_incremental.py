"""Incremental state forking (Flide, "Accelerating Decision Inference with
Exact State Forking", section 3.4) against the oracle.

Round 1 runs a request (a trunk plus question branches off its end) and, in the
same pass, saves the state at an internal trunk position m that is neither a
chunk boundary nor a leaf (a state row). Round 2 is the agent's next step: the
trunk's tail after m has changed, more tokens are appended and new questions
fork from the new trunk; it resumes from the saved checkpoint as its initial
state. Round 2's readouts and states must match the oracle run on the whole
concatenated stream (round 1's tokens up to m, then round 2's tokens) from the
original initial state, and the checkpoint must match the oracle's state at m.
"""
import numpy as np
import pytest
import torch

import oracle
from tree_forked_gated_amd import workloads as W

from gpu_helpers import record_margin, rel_l2, say

pytestmark = pytest.mark.gpu


def _trunk_with_questions(L, qs):
    """Local parents: a chain of L tokens, then branches (fork token, length)."""
    par = list(range(-1, L - 1))
    lasts = []
    for ft, bl in qs:
        b0 = len(par)
        par += [ft] + list(range(b0, b0 + bl - 1))
        lasts.append(len(par) - 1)
    return np.array(par, np.int32), np.array(lasts, np.int32)


def _dev(wl):
    f = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda().to(
        torch.bfloat16 if wl.dtype == "bf16" else torch.float32)
    return f(wl.q), f(wl.k), f(wl.v), f(wl.log_gate), f(wl.beta)


def _forward(wl, init, out_rows, state_rows):
    from tree_forked_gated_amd import binding as B
    q, k, v, g, b = _dev(wl)
    cap = B.capacities(wl.parent, wl.seq_start)
    return B.forward(q, k, v, g, b, wl.parent, wl.seq_start, torch.from_numpy(init).cuda(), out_rows=out_rows,
                     state_rows=state_rows, check=True, **cap)


@pytest.mark.parametrize("dtype,D,H,m", [("bf16", 128, 4, 601), ("f32", 32, 2, 370)])
def test_resume_from_checkpoint_matches_whole_stream(dtype, D, H, m):
    rng = np.random.default_rng(7 if dtype == "bf16" else 8)
    L1 = 700 if dtype == "bf16" else 420
    assert m % 64 not in (0, 63) and m < L1 - 1  # internal, mid-chunk, not a leaf
    p1, lasts1 = _trunk_with_questions(L1, [(L1 - 1, 24), (L1 - 1, 9), (L1 - 1, 40)])
    n1 = p1.shape[0]
    v1 = W._values(rng, n1, H, D, D, dtype)
    init = W._init(rng, 1, H, D, D, True)
    wl1 = W.Workload("round1", dtype, p1, np.array([0, n1], np.int32), *v1, init, lasts1,
                     np.concatenate([[m], lasts1]).astype(np.int32))
    say(f"round 1 ({dtype}): T={n1}, checkpoint at {m}")
    r1 = _forward(wl1, init, wl1.out_rows, wl1.state_rows)
    torch.cuda.synchronize()
    ckpt = r1.state[0:1].cpu().numpy()  # [1, H, Dv, Dk] fp32: the state after token m

    # round 2: the changed tail and new tokens continue from m; new questions fork mid-trunk and at its end
    L2 = 350 if dtype == "bf16" else 200
    p2, lasts2 = _trunk_with_questions(L2, [(L2 - 1, 30), (L2 // 2, 17), (5, 64), (L2 - 1, 3)])
    n2 = p2.shape[0]
    v2 = W._values(rng, n2, H, D, D, dtype)
    wl2 = W.Workload("round2", dtype, p2, np.array([0, n2], np.int32), *v2, ckpt, lasts2,
                     np.concatenate([lasts2, [L2 - 1]]).astype(np.int32))
    say(f"round 2 ({dtype}): T={n2}, resumed from the checkpoint")
    r2 = _forward(wl2, ckpt, wl2.out_rows, wl2.state_rows)
    torch.cuda.synchronize()

    # the oracle on the whole concatenated stream: round 1 up to m, then round 2 hanging off m
    keep = m + 1
    parent = np.concatenate([p1[:keep], np.where(p2 < 0, m, p2 + keep)]).astype(np.int32)
    cat = lambda a, b: np.concatenate([a[:keep], b])
    whole = W.Workload("whole", dtype, parent, np.array([0, keep + n2], np.int32),
                       *(cat(a, b) for a, b in zip(v1, v2)), init, None,
                       np.concatenate([[m], lasts2 + keep, [L2 - 1 + keep]]).astype(np.int32))
    ref = oracle.forward(whole, "f64", state_rows=whole.state_rows)
    tol = 1e-2 if dtype == "bf16" else 1e-4
    errs = {"checkpoint": rel_l2(ckpt, ref["state"][0:1]),
            "out": rel_l2(r2.out.float().cpu().numpy(), ref["out"][lasts2 + keep]),
            "state": rel_l2(r2.state.cpu().numpy(), ref["state"][1:])}
    say(f"  rel-L2 vs the whole stream: {errs}")
    record_margin(f"incremental/{dtype}", tol=tol, **errs)
    for k_, e in errs.items():
        assert e <= tol, (k_, e)
