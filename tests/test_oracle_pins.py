"""Pins of the oracle to facts outside itself (CPU only).

Each test names the fact it checks. Together they are meant to catch a dropped
term, a wrong sign, a wrong index or a transposed operand anywhere in the
oracle's walk: closed forms (pure decay, scalar hand example), invariants
(delta write, fork exactness, sibling isolation, relabelling), a special case
that reduces to a textbook masked matmul (orthonormal keys), and the pages' own
check (closed form Eq. 2/3 against the per-node recurrence).
"""
import json
import os

import numpy as np
import pytest

import oracle
from oracle import closed_form as cf
from tree_forked_gated_amd import workloads as W

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _path_logsum(parent, log_gate, t, h):
    s = 0.0
    while t >= 0:
        s += float(log_gate[t, h])
        t = int(parent[t])
    return s


def _ancestors(parent, t):
    out = set()
    while t >= 0:
        out.add(int(t))
        t = int(parent[t])
    return out


def _seq_of(wl, t):
    return int(np.searchsorted(wl.seq_start, t, side="right") - 1)


def _rel(a, b):
    return float(np.linalg.norm((a - b).ravel()) / max(np.linalg.norm(np.asarray(b).ravel()), 1e-300))


# ---------------------------------------------------------------- hand example

def test_scalar_hand_example():
    """Hand-derived values from Eq. 1 with d_k = d_v = 1 (tests/golden)."""
    g = json.load(open(os.path.join(GOLD, "scalar_tree.json")))
    T = len(g["parent"])
    sh = lambda x: np.array(x, dtype=np.float64).reshape(T, 1, 1)
    wl = W.Workload("scalar", "f32", np.array(g["parent"], np.int32), np.array(g["seq_start"], np.int32),
                    sh(g["q"]), sh(g["k"]), sh(g["v"]), np.array(g["beta"]).reshape(T, 1),
                    np.log(np.array(g["alpha"])).reshape(T, 1), np.full((1, 1, 1, 1), g["init_state"]), None,
                    np.arange(T, dtype=np.int32))
    r = oracle.forward(wl, "f64")
    np.testing.assert_allclose(r["out"].ravel(), g["expected_out"], rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(r["state"].ravel(), g["expected_state"], rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(r["pseudo_v"].ravel(), g["expected_pseudo"], rtol=1e-14, atol=1e-15)


# ---------------------------------------------------------------- closed forms

@pytest.mark.parametrize("seed", [1, 2])
def test_beta_zero_is_pure_decay(seed):
    """beta = 0: S_t = exp(G_t) S_0 with G_t the path sum of log gates, so
    o_t = exp(G_t) S_0 q_t (the erase and write terms vanish)."""
    wl = W.random_small(seed, n_seq=3, H=2, Dk=8, Dv=6, max_len=90)
    wl.beta[:] = 0.0
    r = oracle.forward(wl, "f64", state_rows=np.arange(wl.T, dtype=np.int32))
    for t in range(wl.T):
        s = _seq_of(wl, t)
        for h in range(wl.H):
            G = _path_logsum(wl.parent, wl.log_gate, t, h)
            S = np.exp(G) * wl.init_state[s, h].astype(np.float64)
            np.testing.assert_allclose(r["state"][t, h], S, rtol=1e-13, atol=1e-300)
            np.testing.assert_allclose(r["out"][t, h], S @ wl.q[t, h].astype(np.float64), rtol=1e-12, atol=1e-15)


@pytest.mark.parametrize("seed", [3, 4])
def test_delta_write_recalls_value(seed):
    """beta = 1 with a unit key: the delta rule overwrites what the state
    stores for k_t, so S_t k_t = v_t whatever alpha_t and the parent state."""
    wl = W.random_small(seed, n_seq=3, H=2, Dk=16, Dv=5, max_len=80)
    wl.beta[:] = 1.0
    k64 = wl.k.astype(np.float64)
    wl.k = k64 / np.linalg.norm(k64, axis=-1, keepdims=True)  # unit to fp64 rounding
    r = oracle.forward(wl, "f64", state_rows=np.arange(wl.T, dtype=np.int32))
    recalled = np.einsum("thvd,thd->thv", r["state"], wl.k)
    np.testing.assert_allclose(recalled, wl.v, rtol=0, atol=1e-12)
    # and the pseudo-value of an empty parent state is the value itself times beta
    roots = np.nonzero(wl.parent < 0)[0]
    wl2 = W.random_small(seed, n_seq=3, H=2, Dk=16, Dv=5, max_len=80, random_init=False)
    r2 = oracle.forward(wl2, "f64")
    np.testing.assert_allclose(r2["pseudo_v"][roots], wl2.beta[roots][..., None].astype(np.float64) * wl2.v[roots], rtol=1e-15)


@pytest.mark.parametrize("seed", [5, 6, 7])
def test_orthonormal_keys_give_masked_decayed_attention(seed):
    """Distinct one-hot keys (at most d_k tokens per sequence) and S_0 = 0:
    the erase term never touches other tokens' writes, so
    o_t = sum over i ancestor-or-self of t of exp(G_t - G_i) beta_i (q_t . k_i) v_i,
    i.e. one masked, decayed linear-attention matmul."""
    rng = np.random.default_rng(seed)
    Dk, Dv, H = 48, 7, 2
    lp = W.random_draft_tree(rng, 40, max_depth=6, max_fanout=4)
    T = lp.shape[0]
    base = W.random_small(seed, n_seq=1, H=H, Dk=Dk, Dv=Dv)
    k = np.zeros((T, H, Dk), np.float64)
    for h in range(H):
        perm = rng.permutation(Dk)[:T]
        k[np.arange(T), h, perm] = 1.0
    q = rng.standard_normal((T, H, Dk))
    v = rng.standard_normal((T, H, Dv))
    beta = rng.uniform(0.05, 0.95, (T, H))
    g = -rng.uniform(0.0, 1.5, (T, H))
    wl = W.Workload("ortho", "f32", lp.astype(np.int32), np.array([0, T], np.int32), q, k, v, beta, g,
                    np.zeros((1, H, Dv, Dk)), None, np.zeros(0, np.int32))
    r = oracle.forward(wl, "f64")
    for h in range(H):
        G = np.array([_path_logsum(lp, g, t, h) for t in range(T)])
        mask = np.zeros((T, T))
        for t in range(T):
            for i in _ancestors(lp, t):
                mask[t, i] = np.exp(G[t] - G[i]) * beta[i, h]
        ref = (mask * (q[:, h] @ k[:, h].T)) @ v[:, h]
        np.testing.assert_allclose(r["out"][:, h], ref, rtol=1e-12, atol=1e-12)


# ------------------------------------------------ the pages' check: Eq. 2 / 3

@pytest.mark.parametrize("seed", [8, 9, 10, 11])
def test_closed_form_matches_walk_fp64(seed):
    """TreeWY section 4: the closed form (one triangular solve, Eq. 2; states by
    Eq. 3) equals the per-node recurrence to ~1e-15 in fp64."""
    wl = W.random_small(seed, n_seq=3, H=2, Dk=12, Dv=9, max_len=70)
    rows = np.arange(wl.T, dtype=np.int32)
    r = oracle.forward(wl, "f64", state_rows=rows)
    for s in range(wl.n_seq):
        a, b = int(wl.seq_start[s]), int(wl.seq_start[s + 1])
        if a == b:
            continue
        lp = np.where(wl.parent[a:b] < 0, -1, wl.parent[a:b] - a)
        for h in range(wl.H):
            o, pv, st = cf.tree_wy(lp, wl.q[a:b, h], wl.k[a:b, h], wl.v[a:b, h], wl.beta[a:b, h],
                                   wl.log_gate[a:b, h], wl.init_state[s, h])
            assert _rel(r["out"][a:b, h], o) < 1e-12
            assert _rel(r["pseudo_v"][a:b, h], pv) < 1e-12
            assert _rel(r["state"][a:b, h], st) < 1e-12


def test_closed_form_matches_walk_fp32():
    """Same check for the fp32 build: the pages report ~1e-7 for fp32."""
    wl = W.tiny_tree()
    r = oracle.forward(wl, "f32")
    lp = wl.parent
    o, pv, _ = cf.tree_wy(lp, wl.q[:, 0], wl.k[:, 0], wl.v[:, 0], wl.beta[:, 0], wl.log_gate[:, 0],
                          wl.init_state[0, 0])
    assert _rel(r["out"][:, 0].astype(np.float64), o) < 2e-6
    assert _rel(r["pseudo_v"][:, 0].astype(np.float64), pv) < 2e-6


def test_chain_matches_matrix_form_of_eq1():
    """On a chain the walk equals Eq. 1 written with the explicit transition
    alpha (I - beta k k^T) (a different order of operations)."""
    wl = W.chains(n_seq=1, L=40, H=2, D=8)
    r = oracle.forward(wl, "f64")
    for h in range(wl.H):
        S = wl.init_state[0, h].astype(np.float64)
        for t in range(wl.T):
            kk = wl.k[t, h].astype(np.float64)
            a = np.exp(np.float64(wl.log_gate[t, h]))
            b = np.float64(wl.beta[t, h])
            S = a * S @ (np.eye(8) - b * np.outer(kk, kk)) + b * np.outer(wl.v[t, h], kk)
            np.testing.assert_allclose(r["out"][t, h], S @ wl.q[t, h], rtol=1e-11, atol=1e-13)


# -------------------------------------------------------- fork exactness etc.

def _branch_alone(wl, r_states, fork_tok, branch):
    """A workload holding only `branch` (global ids, parents inside it or
    fork_tok) run from the oracle's state at fork_tok."""
    idx = {t: i for i, t in enumerate(branch)}
    lp = np.array([(-1 if wl.parent[t] == fork_tok else idx[int(wl.parent[t])]) for t in branch], np.int32)
    sl = np.array(branch)
    return W.Workload("alone", wl.dtype, lp, np.array([0, len(branch)], np.int32), wl.q[sl], wl.k[sl], wl.v[sl],
                      wl.beta[sl], wl.log_gate[sl], r_states[None], None, np.zeros(0, np.int32))


@pytest.mark.parametrize("prec", ["f64", "f32"])
def test_fork_exactness_bitwise(prec):
    """Flide Prop. 3.1: a branch inside the tree computes exactly what it
    computes alone from its trunk's state (bitwise in the oracle)."""
    wl = W.tiny_tree()
    r = oracle.forward(wl, prec, state_rows=np.array([15, 31], np.int32))
    for fork, branch in [(31, list(range(40, 48))), (31, list(range(56, 64))), (15, list(range(64, 68))),
                         (31, list(range(32, 40)))]:
        st = r["state"][0 if fork == 15 else 1]
        alone = _branch_alone(wl, st, fork, branch)
        ra = oracle.forward(alone, prec)
        assert np.array_equal(ra["out"], r["out"][branch]), (fork, branch[0])


def test_dfs_relabel_invariance():
    """Another DFS pre-order of the same tree gives every node the same bits."""
    rng = np.random.default_rng(12)
    lp = W.random_draft_tree(rng, 50)
    T = lp.shape[0]
    children = {u: [] for u in range(-1, T)}
    for u in range(T):
        children[int(lp[u])].append(u)
    order, stack = [], list(children[-1])  # reversed sibling order
    while stack:
        u = stack.pop()
        order.append(u)
        stack.extend(children[u])
    new = {u: i for i, u in enumerate(order)}
    base = W.random_small(12, n_seq=1, H=2, Dk=16, Dv=16)
    q, k, v = (rng.standard_normal((T, 2, 16)) for _ in range(3))
    beta, g = rng.uniform(0.1, 0.9, (T, 2)), -rng.uniform(0, 1, (T, 2))
    init = rng.standard_normal((1, 2, 16, 16)) * 0.1
    wl1 = W.Workload("a", "f32", lp, np.array([0, T], np.int32), q, k, v, beta, g, init, None, np.zeros(0, np.int32))
    perm = np.array(order)
    lp2 = np.array([(-1 if lp[u] < 0 else new[int(lp[u])]) for u in order], np.int32)
    wl2 = W.Workload("b", "f32", lp2, np.array([0, T], np.int32), q[perm], k[perm], v[perm], beta[perm], g[perm],
                     init, None, np.zeros(0, np.int32))
    for prec in ("f64", "f32"):
        o1 = oracle.forward(wl1, prec)["out"]
        o2 = oracle.forward(wl2, prec)["out"]
        assert np.array_equal(o1[perm], o2)


def test_no_sibling_leak_and_negative_control():
    """Perturbing sibling branches changes nothing in a branch (bitwise);
    gluing the branch after its siblings as one chain (the delimiter-style
    layout Flide argues against) does change it."""
    wl = W.tiny_tree()
    r = oracle.forward(wl, "f64")
    pert = W.tiny_tree()
    rng = np.random.default_rng(0)
    sib = list(range(40, 64))  # branches 1..3 off token 31
    pert.v[sib] += rng.standard_normal(pert.v[sib].shape)
    pert.k[sib] = np.roll(pert.k[sib], 1, axis=0)
    rp = oracle.forward(pert, "f64")
    keep = list(range(0, 40)) + list(range(64, 68))
    assert np.array_equal(r["out"][keep], rp["out"][keep])
    assert not np.array_equal(r["out"][sib], rp["out"][sib])
    # negative control: branch 3 (56..63) chained after branches 1 and 2
    glued = wl.parent.copy()
    glued[48] = 47
    glued[56] = 55
    wg = W.tiny_tree()
    wg.parent = glued
    rg = oracle.forward(wg, "f64")
    diff = np.abs(rg["out"][56:64] - r["out"][56:64]).max()
    assert diff > 1e-3


def test_commit_replay_matches_eq3_and_forward_state():
    """Commit: replaying the accepted path equals Eq. 3 rebuilt from the
    forward's pseudo-values, and equals the forward's own state at the node."""
    wl = W.draft_trees(n_seq=4, n_nodes=20, H=2, D=16)
    r = oracle.forward(wl, "f64", state_rows=np.arange(wl.T, dtype=np.int32))
    c = oracle.commit(wl, "f64")
    for p in range(wl.n_path):
        nodes = wl.path_nodes[wl.path_ptr[p]:wl.path_ptr[p + 1]]
        s = int(wl.path_seq[p])
        for h in range(wl.H):
            eq3 = cf.commit_state(nodes, None, wl.k[:, h], r["pseudo_v"][:, h], wl.log_gate[:, h], wl.init_state[s, h])
            assert _rel(c[p, h], eq3) < 1e-12
            assert np.array_equal(c[p, h], r["state"][nodes[-1], h])


def test_commit_empty_path_is_initial_state():
    wl = W.draft_trees(n_seq=2, n_nodes=10, H=1, D=16)
    c = oracle.commit(wl, "f64", path_ptr=np.array([0, 0], np.int32), path_nodes=np.zeros(0, np.int32),
                      path_seq=np.array([1], np.int32))
    assert np.array_equal(c[0], wl.init_state[1])


def test_oracle_rejects_bad_structure():
    wl = W.tiny_tree()
    wl.parent = wl.parent.copy()
    wl.parent[10] = 10
    with pytest.raises(ValueError):
        oracle.forward(wl, "f64")
    wl = W.draft_trees(n_seq=2, n_nodes=10, H=1, D=16)
    with pytest.raises(ValueError):
        oracle.commit(wl, "f64", path_ptr=np.array([0, 1], np.int32), path_nodes=np.array([12], np.int32),
                      path_seq=np.array([0], np.int32))
