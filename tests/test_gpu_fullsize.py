"""HIP path vs the fp64 oracle at full size, plus the boundary cases of the
chunking.

Full size: the four streams the bench times, at their full sizes and in the
bench's launch configuration (automatic d_v tile, one workgroup per CU), each
compared element by element with the oracle over every output. Besides the
relative L2 of each tensor (1e-2 for bf16 inputs), every (token, head) row of
the output and every state must stay within 5e-2 of the typical row norm, so
that a wrong row cannot hide in a global norm.

Boundaries: sequences of 1, 63, 64, 65, 127, 128 and 129 tokens (a whole tree
chunk, a chain of one chunk and a one-token tail), an empty sequence in the
middle of the stream, forks from the last token of a chunk and from the first
token of the next, and an empty stream.
"""
import numpy as np
import pytest
import torch

from tree_forked_gated_amd import workloads as W

from gpu_helpers import f64, oracle_ref, record_margin, rel_l2, run_forward, say, tol

pytestmark = pytest.mark.gpu

ROW_TOL = 5e-2


def _rows_ok(gpu, ref, what):
    """Largest error of one row (last axis, or last two for states) relative to
    the root-mean-square row norm of the reference."""
    g = np.asarray(gpu, np.float64)
    r = np.asarray(ref, np.float64)
    axes = (-1,) if g.ndim == 3 else (-2, -1)
    err = np.sqrt(np.sum((g - r) ** 2, axis=axes))
    scale = np.sqrt(np.mean(np.sum(r ** 2, axis=axes)))
    worst = float(err.max() / max(scale, 1e-30))
    say(f"  {what}: worst row error {worst:.3e} of the typical row norm")
    assert worst <= ROW_TOL, (what, worst)
    return worst


@pytest.mark.parametrize("name", ["chains", "decision_round", "draft_trees", "mixed_forest"])
def test_full_size_against_oracle(name):
    wl = W.get(name)
    rows = wl.state_rows if wl.state_rows.size else W.leaves_of(wl.parent)
    say(f"full size {wl.name}: T={wl.T} H={wl.H} seqs={wl.n_seq} states={rows.shape[0]}")
    res, d = run_forward(wl, keep_pseudo=wl.keep_pseudo, state_rows=rows)
    ref = oracle_ref(wl, state_rows=rows, keep_pseudo=wl.keep_pseudo)
    ref_out = ref["out"] if wl.out_rows is None else ref["out"][wl.out_rows]
    out = f64(res.out)
    st = f64(res.state)
    errs = {"out": rel_l2(out, ref_out), "state": rel_l2(st, ref["state"])}
    if wl.keep_pseudo:
        errs["pseudo_v"] = rel_l2(f64(res.pseudo_v), ref["pseudo_v"])
    say(f"  rel-L2 {errs}")
    worst = {"out_worst_row": _rows_ok(out, ref_out, "out"), "state_worst_row": _rows_ok(st, ref["state"], "state")}
    record_margin(f"full_size/{wl.name}", tol=tol(wl), row_tol=ROW_TOL, **errs, **worst)
    for k, e in errs.items():
        assert e <= tol(wl), (name, k, e)
    if wl.path_ptr is not None:  # draft trees: commit the accepted paths
        import oracle
        from tree_forked_gated_amd import binding as B
        got = B.commit(d["k"], d["log_gate"], d["parent_idx"], d["seq_start"], d["init_state"], res.pseudo_v,
                       wl.path_ptr, wl.path_nodes, wl.path_seq, check=True)
        torch.cuda.synchronize()
        refc = oracle.commit(wl, "f64")
        e = rel_l2(f64(got), refc)
        say(f"  commit rel-L2 {e:.3e}")
        wc = _rows_ok(f64(got), refc, "commit")
        record_margin(f"full_size/{wl.name}/commit", tol=tol(wl), commit=e, commit_worst_row=wc)
        assert e <= tol(wl)


def _stream(lens, forks=(), H=3, D=128, seed=77):
    """Chains of the given lengths (0 = empty sequence) in one stream; forks are
    (sequence, token within it, branch length): a branch appended to that
    sequence whose first token's parent is the given token."""
    rng = np.random.default_rng(seed)
    parents, starts, used = [], [0], 0
    for s, L in enumerate(lens):
        par = list(range(-1, L - 1)) if L else []
        for fs, ft, bl in forks:
            if fs == s:
                b0 = len(par)
                par += [ft] + list(range(b0, b0 + bl - 1))
        parents.append(np.array([p + used if p >= 0 else -1 for p in par], dtype=np.int32))
        used += len(par)
        starts.append(used)
    parent = np.concatenate(parents) if used else np.zeros(0, np.int32)
    seq_start = np.array(starts, dtype=np.int32)
    T, n_seq = int(parent.shape[0]), len(lens)
    q, k, v, beta, g = W._values(rng, T, H, D, D, "bf16")
    init = W._init(rng, n_seq, H, D, D, True)
    return W.Workload(f"boundary_{T}", "bf16", parent, seq_start, q, k, v, beta, g, init, None,
                      W.leaves_of(parent))


@pytest.mark.parametrize("dv_tile", [0, 16, 64])
def test_chunk_boundaries(dv_tile):
    wl = _stream([1, 63, 64, 0, 65, 127, 128, 129, 200],
                 forks=[(8, 63, 40), (8, 64, 70), (7, 127, 3), (6, 126, 65)])
    say(f"boundaries: T={wl.T} seqs={wl.n_seq} dv_tile={dv_tile}")
    res, _ = run_forward(wl, keep_pseudo=True, dv_tile=dv_tile)
    ref = oracle_ref(wl)
    errs = {"out": rel_l2(f64(res.out), ref["out"]), "state": rel_l2(f64(res.state), ref["state"]),
            "pseudo_v": rel_l2(f64(res.pseudo_v), ref["pseudo_v"])}
    say(f"  rel-L2 {errs}")
    for k, e in errs.items():
        assert e <= tol(wl), (k, e)
    _rows_ok(f64(res.out), ref["out"], "out")
    _rows_ok(f64(res.state), ref["state"], "state")


def test_empty_stream():
    from tree_forked_gated_amd import binding as B
    say("empty stream")
    dev = "cuda"
    e = lambda *s: torch.empty(s, dtype=torch.bfloat16, device=dev)
    res = B.forward(e(0, 2, 128), e(0, 2, 128), e(0, 2, 128), e(0, 2), e(0, 2),
                    torch.zeros(0, dtype=torch.int32, device=dev), torch.zeros(2, dtype=torch.int32, device=dev),
                    torch.zeros((1, 2, 128, 128), dtype=torch.float32, device=dev), max_forks=0, max_levels=1,
                    check=True)
    torch.cuda.synchronize()
    assert res.out.shape[0] == 0
