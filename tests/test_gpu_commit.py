"""gdn_tree_commit against the oracle's replay of the accepted paths.

The commit rebuilds the state after each accepted path from the initial state
and the forward's pseudo-values (TreeWY, "Speculative Verification for Gated
DeltaNet Hybrids", section 3, Eq. 3); the oracle replays the recurrence along
the same path token by token. Cases: empty paths (the initial state), paths of
a root alone, paths to internal nodes and to leaves, paths of 100-200 nodes
(many 16-node tiles and a ragged last tile), several paths per sequence, d_v
blocks of 16 rows after blocks of 32 (d_v = 48 and 80), no initial states, fp32
and bf16. Tolerances: relative L2 1e-4 (fp32) and 1e-2 (bf16) per tensor.

Error cases: a path that skips a node, a path whose node lies in another
sequence, node indices outside [0, T), a path whose sequence index is out of
range each raise the path error with the
smallest bad path's index, both when one workgroup decides the error word (up
to 1024 paths) and when the workgroups raise it by atomics (more paths); the
states of the good paths are still written and still match the oracle. Zero paths
enqueue nothing but the error word's reset.
"""
import numpy as np
import pytest
import torch

import oracle
from tree_forked_gated_amd import workloads as W

from gpu_helpers import f64, record_margin, rel_l2, run_forward, say, tol

pytestmark = pytest.mark.gpu

DEV_PATH = 7  # GDN_DEV_PATH


def _workload(seed, dtype, Dk, Dv, random_init=True):
    wl = W.random_small(seed, n_seq=6, H=3, Dk=Dk, Dv=Dv, dtype=dtype, max_len=200, random_init=random_init)
    wl.keep_pseudo = True
    return wl


def _paths(wl, rng):
    """Per sequence: an empty path, the root alone, a path to a random node and
    to the deepest node; the sequences in shuffled order."""
    ptr, nodes, seqs = [0], [], []
    order = rng.permutation(wl.n_seq)
    for s in order:
        a, b = int(wl.seq_start[s]), int(wl.seq_start[s + 1])
        if b <= a:
            continue
        depth = np.zeros(b - a, np.int64)
        for t in range(a, b):
            p = int(wl.parent[t])
            depth[t - a] = 0 if p < 0 else depth[p - a] + 1
        deepest = a + int(np.argmax(depth))
        for end in (None, a, a + int(rng.integers(0, b - a)), deepest):
            path = [] if end is None else W.root_path(wl.parent, end)
            nodes += path
            ptr.append(len(nodes))
            seqs.append(int(s))
    return np.array(ptr, np.int32), np.array(nodes, np.int32), np.array(seqs, np.int32)


def _commit(d, res, ptr, nodes, seqs, init=True, check=True, workspace=None):
    from tree_forked_gated_amd import binding as B
    got = B.commit(d["k"], d["log_gate"], d["parent_idx"], d["seq_start"], d["init_state"] if init else None,
                   res.pseudo_v, ptr, nodes, seqs, check=check, workspace=workspace)
    torch.cuda.synchronize()
    return got


@pytest.mark.parametrize("dtype,Dk,Dv,seed", [("f32", 64, 48, 11), ("f32", 16, 16, 12), ("bf16", 128, 80, 13),
                                              ("bf16", 32, 16, 14), ("bf16", 64, 128, 15)])
def test_commit_paths_against_oracle(dtype, Dk, Dv, seed):
    wl = _workload(seed, dtype, Dk, Dv)
    ptr, nodes, seqs = _paths(wl, np.random.default_rng(seed))
    lens = np.diff(ptr)
    say(f"commit {dtype} Dk={Dk} Dv={Dv}: T={wl.T}, {lens.size} paths of 0..{lens.max()} nodes")
    assert lens.max() > 48 and (lens == 0).any() and (lens == 1).any()
    res, d = run_forward(wl, keep_pseudo=True, state_rows=W.leaves_of(wl.parent))
    got = _commit(d, res, ptr, nodes, seqs)
    ref = oracle.commit(wl, "f64", path_ptr=ptr, path_nodes=nodes, path_seq=seqs)
    e = rel_l2(f64(got), ref)
    # an empty path commits the initial state exactly
    empty = np.nonzero(lens == 0)[0]
    assert np.array_equal(f64(got)[empty], wl.init_state[seqs[empty]].astype(np.float64))
    say(f"  rel-L2 {e:.3e}")
    record_margin(f"commit/{dtype}_dk{Dk}_dv{Dv}", tol=tol(wl), commit=e)
    assert e <= tol(wl), e


def test_commit_without_initial_states():
    wl = _workload(21, "f32", 32, 48, random_init=False)
    ptr, nodes, seqs = _paths(wl, np.random.default_rng(21))
    res, d = run_forward(wl, keep_pseudo=True, state_rows=W.leaves_of(wl.parent))
    got = _commit(d, res, ptr, nodes, seqs, init=False)
    ref = oracle.commit(wl, "f64", path_ptr=ptr, path_nodes=nodes, path_seq=seqs)
    e = rel_l2(f64(got), ref)
    say(f"commit without initial states: rel-L2 {e:.3e}")
    assert not f64(got)[np.diff(ptr) == 0].any()
    assert e <= tol(wl), e


def _deepest_path(wl, s):
    a, b = int(wl.seq_start[s]), int(wl.seq_start[s + 1])
    return max((W.root_path(wl.parent, t) for t in range(a, b)), key=len, default=[])


def _bad_paths(wl):
    """Good and bad paths mixed: returns ptr, nodes, seqs and the indices of the bad ones."""
    sa, sb = np.argsort([-len(_deepest_path(wl, s)) for s in range(wl.n_seq)])[:2]
    sa, sb = int(sa), int(sb)
    good_a, good_b = _deepest_path(wl, sa), _deepest_path(wl, sb)
    assert len(good_a) > 2 and len(good_b) > 0
    ub = int(wl.seq_start[sb])
    entries = [
        (good_a, sa, True),
        (good_a[:1] + good_a[2:], sa, False),  # skips a node
        (good_b, sb, True),
        (good_a[:2] + [ub], sa, False),        # a node of another sequence
        ([wl.T + 5], sa, False),               # past the stream
        ([-3] + good_a[1:], sa, False),        # a negative index
        (good_b, wl.n_seq + 2, False),         # sequence index out of range
        ([], sb, True),
    ]
    ptr, nodes, seqs, bad = [0], [], [], []
    for i, (path, s, ok) in enumerate(entries):
        nodes += path
        ptr.append(len(nodes))
        seqs.append(s)
        if not ok:
            bad.append(i)
    return ptr, nodes, seqs, bad


@pytest.mark.parametrize("n_lead", [0, 1100])
def test_commit_bad_paths_raise_smallest(n_lead):
    """n_lead 0: 8 paths (one workgroup decides the error word); n_lead 1100:
    1100 good paths first, 1108 in all (the workgroups raise the error word
    by atomics, and the first bad path's index is past 1024)."""
    from tree_forked_gated_amd import binding as B
    wl = _workload(31, "f32", 32, 32)
    ptr, nodes, seqs, bad = _bad_paths(wl)
    n0 = len(seqs)
    good = [i for i in range(n0) if i not in bad]
    idx_map = [good[i % len(good)] for i in range(n_lead)] + list(range(n0))
    P, N, S = [0], [], []
    for i in idx_map:
        N += nodes[ptr[i]:ptr[i + 1]]
        P.append(len(N))
        S.append(seqs[i])
    first_bad = n_lead + bad[0]
    ptr, nodes, seqs = P, N, S
    ptr, nodes, seqs = np.array(ptr, np.int32), np.array(nodes, np.int32), np.array(seqs, np.int32)
    say(f"commit bad paths: {seqs.size} paths, first bad {first_bad}")
    res, d = run_forward(wl, keep_pseudo=True, state_rows=W.leaves_of(wl.parent))
    ws = torch.empty(int(B.lib.gdn_tree_commit_workspace_size()), dtype=torch.uint8, device="cuda")
    got = _commit(d, res, ptr, nodes, seqs, check=False, workspace=ws)
    with pytest.raises(B.GdnDeviceError) as ei:
        B.raise_device_error(ws)
    assert ei.value.code == DEV_PATH and ei.value.index == first_bad, (ei.value.code, ei.value.index)
    # the good paths' states are written all the same
    ok_rows = [i for i, src in enumerate(idx_map) if src in good]
    sub_ptr, sub_nodes = [0], []
    for i in ok_rows:
        sub_nodes += list(nodes[ptr[i]:ptr[i + 1]])
        sub_ptr.append(len(sub_nodes))
    ref = oracle.commit(wl, "f64", path_ptr=np.array(sub_ptr, np.int32), path_nodes=np.array(sub_nodes, np.int32),
                        path_seq=seqs[ok_rows])
    e = rel_l2(f64(got)[ok_rows], ref)
    say(f"  error {ei.value.code} at {ei.value.index}; good paths rel-L2 {e:.3e}")
    assert e <= tol(wl), e


def test_commit_of_no_paths():
    """Zero paths: nothing is computed, the error word reads no error."""
    from tree_forked_gated_amd import binding as B
    wl = _workload(41, "bf16", 64, 32)
    res, d = run_forward(wl, keep_pseudo=True, state_rows=W.leaves_of(wl.parent))
    ws = torch.full((int(B.lib.gdn_tree_commit_workspace_size()),), 255, dtype=torch.uint8, device="cuda")
    got = _commit(d, res, np.zeros(1, np.int32), np.zeros(0, np.int32), np.zeros(0, np.int32), check=False,
                  workspace=ws)
    assert got.shape[0] == 0
    B.raise_device_error(ws)
