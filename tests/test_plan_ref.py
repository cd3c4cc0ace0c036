"""The reference metadata planner against hand-worked trees and brute force."""
import numpy as np
import pytest

from oracle import plan as P
from tree_forked_gated_amd import workloads as W


def test_tiny_tree_plan_by_hand():
    """Config-0 tree: the first branch directly follows the trunk's last token
    (parent = t - 1), so it continues the trunk's segment; the other three
    branches off token 31 and the branch off token 15 start segments."""
    wl = W.tiny_tree()
    p = P.plan(wl.parent, wl.seq_start)
    assert p["error"] == (0, 0)
    assert p["seg_start"].tolist() == [0, 40, 48, 56, 64]
    assert p["seg_len"].tolist() == [40, 8, 8, 8, 4]
    assert p["seg_entry"].tolist() == [-1, 31, 31, 31, 15]
    assert p["seg_mode"].tolist() == [0, 0, 0, 0, 0]
    assert p["seg_level"].tolist() == [0, 1, 1, 1, 1]
    assert p["n_fork"] == 2
    assert p["fork_slot"][15] == 0 and p["fork_slot"][31] == 1
    assert p["seg_slot"].tolist() == [-1, 1, 1, 1, 0]
    exp_depth = list(range(40)) + [32 + i for _ in range(3) for i in range(8)] + [16, 17, 18, 19]
    assert p["depth"].tolist() == exp_depth
    assert p["seg_nchunks"].tolist() == [1, 1, 1, 1, 1]


def test_tree_mode_masks_by_hand():
    # two roots; node 2 under 0, node 3 under 2, node 4 under 1
    parent = np.array([-1, -1, 0, 2, 1], np.int32)
    p = P.plan(parent, np.array([0, 5], np.int32))
    m = p["tree_mask"][0]
    assert [int(x) for x in m[:5]] == [0b00001, 0b00010, 0b00101, 0b01101, 0b10010]
    assert p["seg_mode"].tolist() == [1] and p["seg_entry"].tolist() == [-1] and p["n_fork"] == 0
    assert p["depth"].tolist() == [0, 0, 1, 2, 1]


@pytest.mark.parametrize("seed", range(6))
def test_plan_invariants_random(seed):
    wl = W.random_small(seed, n_seq=5, H=1, Dk=16, Dv=16, max_len=300)
    p = P.plan(wl.parent, wl.seq_start)
    T = wl.T
    assert p["error"] == (0, 0)
    # segments tile [0, T) in order and never cross a sequence boundary
    ends = p["seg_start"] + p["seg_len"]
    assert p["seg_start"][0] == 0 and ends[-1] == T and np.all(ends[:-1] == p["seg_start"][1:])
    for i in range(p["n_seg"]):
        a, b = int(p["seg_start"][i]), int(ends[i])
        s = int(p["seg_seq"][i])
        assert wl.seq_start[s] <= a and b <= wl.seq_start[s + 1]
        if p["seg_mode"][i] == 0:
            # inside a chain segment every token's parent is the token before it
            assert all(wl.parent[t] == t - 1 for t in range(a + 1, b))
            assert p["seg_entry"][i] == wl.parent[a]
        else:
            assert a == wl.seq_start[s] and b == wl.seq_start[s + 1] and b - a <= 64
    # depth by walking up
    for t in range(T):
        d, u = 0, int(wl.parent[t])
        while u >= 0:
            d += 1
            u = int(wl.parent[u])
        assert p["depth"][t] == d
    # level = number of fork hops to an initial state
    seg_of = np.searchsorted(p["seg_start"], np.arange(T), side="right") - 1
    for i in range(p["n_seg"]):
        lv, e = 0, int(p["seg_entry"][i])
        while e >= 0:
            lv += 1
            e = int(p["seg_entry"][seg_of[e]])
        assert p["seg_level"][i] == lv
    # fork slots: exactly the entry tokens, numbered in stream order
    forks = sorted(set(int(e) for e in p["seg_entry"] if e >= 0))
    assert [int(p["fork_slot"][t]) for t in forks] == list(range(len(forks)))
    assert int(np.sum(p["fork_slot"] >= 0)) == len(forks)


@pytest.mark.parametrize("bad,code,idx", [
    ({"parent": {3: 3}}, P.DEV_PARENT_ORDER, 3),
    ({"parent": {5: -2}}, P.DEV_PARENT_ORDER, 5),
    ({"parent": {70: 2}}, P.DEV_PARENT_SEQ, 70),
    ({"seq": {1: 200}}, P.DEV_SEQ_START, 1),
])
def test_plan_errors(bad, code, idx):
    wl = W.draft_trees(n_seq=3, n_nodes=64, H=1, D=16)
    parent = wl.parent.copy()
    seq = wl.seq_start.copy()
    for t, v in bad.get("parent", {}).items():
        parent[t] = v
    for s, v in bad.get("seq", {}).items():
        seq[s] = v
    assert P.plan(parent, seq)["error"] == (code, idx)


def test_plan_capacity_and_rows_errors():
    wl = W.tiny_tree()
    assert P.plan(wl.parent, wl.seq_start, max_forks=1)["error"] == (P.DEV_FORK_CAPACITY, 31)
    assert P.plan(wl.parent, wl.seq_start, max_levels=1)["error"] == (P.DEV_LEVEL_CAPACITY, 40)
    assert P.plan(wl.parent, wl.seq_start, out_rows=np.array([3, 3]))["error"] == (P.DEV_ROWS, 1)
    assert P.plan(wl.parent, wl.seq_start, state_rows=np.array([68]))["error"] == (P.DEV_ROWS, 0)
