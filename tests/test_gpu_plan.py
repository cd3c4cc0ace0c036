"""GPU metadata is bit-exact against the reference planner (oracle/plan.py)."""
import numpy as np
import pytest

from oracle import plan as P
from tree_forked_gated_amd import workloads as W

from gpu_helpers import say

pytestmark = pytest.mark.gpu


def _compare(parent, seq_start, **kw):
    from tree_forked_gated_amd import binding as B
    ref = P.plan(parent, seq_start, max_forks=kw.get("max_forks"), max_levels=kw.get("max_levels"),
                 out_rows=kw.get("out_rows"), state_rows=kw.get("state_rows"))
    got = B.plan(parent, seq_start, **kw)
    assert tuple(int(x) for x in got["error"]) == tuple(ref["error"]), (got["error"], ref["error"])
    if ref["error"] != (0, 0):
        return got, ref
    assert got["n_seg"] == ref["n_seg"] and got["n_fork"] == ref["n_fork"]
    for f in ["tok_seq", "depth", "fork_slot"]:
        assert np.array_equal(got[f], ref[f]), f
    for f in ["seg_start", "seg_len", "seg_seq", "seg_mode", "seg_entry", "seg_slot", "seg_level"]:
        assert np.array_equal(got[f], ref[f]), f
    assert np.array_equal(got["tree_mask"], ref["tree_mask"])
    # levels: the set of segments of every level, listed longest first by chunk
    # count (counts of 63 and more tie; order among ties is unspecified)
    ptr = got["level_ptr"]
    nch = np.where(ref["seg_mode"] == 1, 1, (ref["seg_len"] + 63) // 64)
    for lv in range(len(got["level_count"])):
        lst = got["level_items"][ptr[lv]:ptr[lv + 1]]
        assert sorted(lst.tolist()) == np.nonzero(ref["seg_level"] == lv)[0].tolist()
        key = np.minimum(nch[lst], 63)
        assert np.all(key[:-1] >= key[1:]), (lv, key.tolist())
    return got, ref


def _trees(sizes, seed=5):
    """Draft trees of the given sizes (0 for an empty sequence), local parents."""
    rng = np.random.default_rng(seed)
    parents, starts, used = [], [0], 0
    for n in sizes:
        lp = W.random_draft_tree(rng, n) if n else np.zeros(0, np.int32)
        parents.append(np.where(lp < 0, -1, lp + used).astype(np.int32))
        used += n
        starts.append(used)
    return np.concatenate(parents).astype(np.int32), np.array(starts, np.int32)


def test_plan_short_sequences_with_rows():
    """The one-pass path: every sequence fits one chunk (empty and one-token
    sequences among them), with readout and state rows."""
    parent, seq = _trees([64, 1, 0, 37, 64, 2, 17, 50, 1, 0])
    T = parent.shape[0]
    rng = np.random.default_rng(6)
    say(f"plan short sequences T={T}")
    got, _ = _compare(parent, seq, out_rows=rng.permutation(T)[:90].astype(np.int32),
                      state_rows=rng.permutation(T)[:40].astype(np.int32))
    assert got["n_fork"] == 0 and got["n_seg"] == 8


def test_plan_tiny_tree():
    wl = W.tiny_tree()
    say("plan tiny_tree")
    got, _ = _compare(wl.parent, wl.seq_start)
    assert got["seg_start"].tolist() == [0, 40, 48, 56, 64]


@pytest.mark.parametrize("seed", range(8))
def test_plan_random(seed):
    wl = W.random_small(seed, n_seq=7, H=1, Dk=16, Dv=16, max_len=400)
    say(f"plan random_small seed={seed} T={wl.T}")
    _compare(wl.parent, wl.seq_start)


def test_plan_draft_trees_and_forests():
    wl = W.draft_trees(n_seq=16, n_nodes=64, H=1, D=32)
    say("plan draft_trees structure")
    _compare(wl.parent, wl.seq_start)
    wl = W.mixed_forest(total=20000, H=1, D=32)
    say(f"plan mixed_forest-shaped structure T={wl.T}")
    _compare(wl.parent, wl.seq_start)


def test_plan_full_size_structures():
    for name in ["decision_round", "mixed_forest"]:
        wl = W.get(name, H=1, D=32)
        say(f"plan full-size structure {name} T={wl.T}")
        _compare(wl.parent, wl.seq_start)


@pytest.mark.parametrize("case", ["order", "self", "below", "crossseq", "seqstart", "seqlast", "noseq", "forkcap",
                                  "levelcap", "rowdup", "rowrange"])
@pytest.mark.parametrize("shape", ["mixed", "long", "trees"])
def test_plan_errors_match(case, shape):
    """Short streams are planned by one workgroup (in one pass when every
    sequence fits one chunk), long ones by six launches: all report the same
    first error as the reference planner."""
    if shape == "trees":
        parent, seq = _trees([9, 30, 0, 64, 5, 1])
    else:
        wl = W.random_small(11, n_seq=4, H=1, Dk=16, Dv=16, max_len=200)
        parent = wl.parent.copy()
        seq = wl.seq_start.copy()
    if shape == "long":  # a 5000-token chain appended as a fifth sequence
        T0 = wl.T
        chain = np.arange(T0 - 1, T0 + 4999, dtype=np.int32)
        chain[0] = -1
        parent = np.concatenate([parent, chain]).astype(np.int32)
        seq = np.concatenate([seq, [T0 + 5000]]).astype(np.int32)
    kw = {}
    T = int(parent.shape[0])
    if case == "order":
        parent[T - 3] = T - 1
    elif case == "self":
        parent[5] = 5
    elif case == "below":
        parent[7] = -5
    elif case == "crossseq":
        t = int(seq[2]) + 1
        parent[t] = int(seq[1]) - 1
    elif case == "seqstart":
        seq[2] = seq[1] - 1
    elif case == "seqlast":
        seq[-1] = T - 1
    elif case == "noseq":  # no sequence at all, but T > 0 tokens
        seq = np.zeros(1, np.int32)
        kw = {"max_forks": 0, "max_levels": 1}
    elif case == "forkcap":
        ref = P.plan(parent, seq)
        kw = {"max_forks": max(0, ref["n_fork"] - 1), "max_levels": 64}
    elif case == "levelcap":
        ref = P.plan(parent, seq)
        kw = {"max_forks": ref["n_fork"], "max_levels": max(1, ref["n_levels"] - 1)}
    elif case == "rowdup":
        kw = {"out_rows": np.array([1, 2, 1], np.int32)}
    elif case == "rowrange":
        kw = {"state_rows": np.array([0, T], np.int32)}
    say(f"plan error case {case} shape={shape} T={T}")
    got, ref = _compare(parent, seq, **kw)
    if case not in ("forkcap", "levelcap") or ref["error"] != (0, 0):
        assert ref["error"] != (0, 0)
