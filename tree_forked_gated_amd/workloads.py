"""Seeded synthetic tree streams for the tree-structured gated delta rule.

This module only draws inputs: tree structures, q/k/v, write strengths, log
gates, initial states and commit paths. It holds none of the recurrence's
arithmetic and is shared by the tests, the bench and the oracle's callers.

Shapes follow the two workloads of the pages:

* decision rounds (Flide, "Accelerating Decision Inference with Exact State
  Forking", sections 3.3 and 4.1): long shared trunks with short question
  branches forking from them, laid out trunk first;
* speculative draft trees (TreeWY, "Speculative Verification for Gated
  DeltaNet Hybrids", section 3 "Verifying a draft"): small trees over a
  committed state, laid out in DFS pre-order, then one accepted root-to-node
  path to commit.

Value recipe (all workloads): q and k are standard normal, then L2-normalised
per (token, head) in fp32; v is standard normal; beta = sigmoid(N(0,1));
log_gate = -softplus(N(0,1)); initial states are N(0, 0.02^2) where a workload
asks for them, zeros otherwise. Every array is drawn as fp64 standard normal in
C order from numpy's PCG64 seeded generator, cast to fp32, and for bf16
workloads rounded to bf16 (round to nearest even). The arrays returned hold the
rounded values, so every consumer sees exactly the same numbers.
"""
from __future__ import annotations

import dataclasses
from typing import List, Optional

import numpy as np

CHUNK = 64  # documented here only to size workloads; the kernels own their tiling


# --------------------------------------------------------------------------- bf16

def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to the nearest bf16 (ties to even); returns fp32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    if not np.all(np.isfinite(x)):
        raise ValueError("bf16_round expects finite values")
    u = x.view(np.uint32)
    # finite values stay below 0xFF800000 after the rounding increment, so
    # 32-bit arithmetic cannot wrap
    r = (u >> 16) & np.uint32(1)
    r += u
    r += np.uint32(0x7FFF)
    r &= np.uint32(0xFFFF0000)
    return r.view(np.float32).reshape(x.shape)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Raw bf16 bit patterns (uint16) of values that are already bf16-exact."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    assert np.all((u & 0xFFFF) == 0), "values are not bf16-exact"
    return (u >> 16).astype(np.uint16)


# ------------------------------------------------------------------- container

@dataclasses.dataclass
class Workload:
    name: str
    dtype: str                      # "f32" or "bf16": dtype of q, k, v, beta, log_gate and out
    parent: np.ndarray              # int32 [T]  global index of the parent, -1 = sequence init state
    seq_start: np.ndarray           # int32 [n_seq + 1]
    q: np.ndarray                   # float32 [T, H, Dk] (bf16-exact for bf16 workloads)
    k: np.ndarray                   # float32 [T, H, Dk]
    v: np.ndarray                   # float32 [T, H, Dv]
    beta: np.ndarray                # float32 [T, H]
    log_gate: np.ndarray            # float32 [T, H]
    init_state: np.ndarray          # float32 [n_seq, H, Dv, Dk]
    out_rows: Optional[np.ndarray]  # int32 [n_out] or None (= every token)
    state_rows: np.ndarray          # int32 [n_state]
    keep_pseudo: bool = False
    path_ptr: Optional[np.ndarray] = None    # int32 [n_path + 1]
    path_nodes: Optional[np.ndarray] = None  # int32 [sum of path lengths]
    path_seq: Optional[np.ndarray] = None    # int32 [n_path]
    info: dict = dataclasses.field(default_factory=dict)

    @property
    def T(self) -> int:
        return int(self.parent.shape[0])

    @property
    def H(self) -> int:
        return int(self.q.shape[1])

    @property
    def Dk(self) -> int:
        return int(self.q.shape[2])

    @property
    def Dv(self) -> int:
        return int(self.v.shape[2])

    @property
    def n_seq(self) -> int:
        return int(self.seq_start.shape[0] - 1)

    @property
    def n_path(self) -> int:
        return 0 if self.path_ptr is None else int(self.path_ptr.shape[0] - 1)


# ------------------------------------------------------------ structure helpers

def leaves_of(parent: np.ndarray) -> np.ndarray:
    """Tokens that no other token names as parent, in stream order."""
    has_child = np.zeros(parent.shape[0], dtype=bool)
    p = parent[parent >= 0]
    has_child[p] = True
    return np.nonzero(~has_child)[0].astype(np.int32)


def root_path(parent: np.ndarray, node: int) -> List[int]:
    """Global indices from the root of `node` down to `node` itself."""
    out = []
    while node >= 0:
        out.append(int(node))
        node = int(parent[node])
    return out[::-1]


def _normal_f32(rng, shape, unit_rows=False, rows_per_block=2048):
    """Standard normal fp64 draws in C order, cast to fp32 (and L2-normalised
    along the last axis in fp32 when unit_rows). Drawn block by block along the
    first axis: the generator yields the same numbers in the same order as one
    draw of the whole shape, without a multi-gigabyte fp64 temporary."""
    out = np.empty(shape, dtype=np.float32)
    n = shape[0] if len(shape) else 0
    for a in range(0, n, rows_per_block):
        b = min(n, a + rows_per_block)
        blk = rng.standard_normal((b - a,) + tuple(shape[1:])).astype(np.float32)
        if unit_rows:
            nrm = np.sqrt(np.sum(blk * blk, axis=-1, keepdims=True, dtype=np.float32), dtype=np.float32)
            blk = (blk / nrm).astype(np.float32)
        out[a:b] = blk
    return out


def _values(rng, T, H, Dk, Dv, dtype):
    """Draw q, k, v, beta, log_gate in the documented order and recipe."""
    q = _normal_f32(rng, (T, H, Dk), unit_rows=True)
    k = _normal_f32(rng, (T, H, Dk), unit_rows=True)
    v = _normal_f32(rng, (T, H, Dv))
    xb = rng.standard_normal((T, H))
    beta = (1.0 / (1.0 + np.exp(-xb))).astype(np.float32)
    xg = rng.standard_normal((T, H))
    log_gate = (-np.logaddexp(0.0, xg)).astype(np.float32)
    if dtype == "bf16":
        q, k, v, beta, log_gate = (bf16_round(a) for a in (q, k, v, beta, log_gate))
    return q, k, v, beta, log_gate


def _init(rng, n_seq, H, Dv, Dk, random_init):
    if random_init:
        return (0.02 * rng.standard_normal((n_seq, H, Dv, Dk))).astype(np.float32)
    return np.zeros((n_seq, H, Dv, Dk), dtype=np.float32)


# --------------------------------------------------------------------- configs

def tiny_tree(seed: int = 1000) -> Workload:
    """Tiny fp32 tree: trunk of 32, four 8-token branches off the trunk's last
    token, one 4-token branch off trunk token 15 (0-based stream index)."""
    rng = np.random.default_rng(seed)
    H, D = 1, 16
    parent = []
    for t in range(32):
        parent.append(t - 1)
    for b in range(4):
        base = 32 + 8 * b
        for i in range(8):
            parent.append(31 if i == 0 else base + i - 1)
    for i in range(4):
        parent.append(15 if i == 0 else 64 + i - 1)
    parent = np.array(parent, dtype=np.int32)
    T = parent.shape[0]
    seq_start = np.array([0, T], dtype=np.int32)
    q, k, v, beta, g = _values(rng, T, H, D, D, "f32")
    init = _init(rng, 1, H, D, D, False)
    return Workload("tiny_tree_f32", "f32", parent, seq_start, q, k, v, beta, g, init,
                    None, leaves_of(parent), info={"structure": "trunk 32 + 4x8 off 31 + 4 off 15"})


def chains(seed: int = 1001, n_seq: int = 4, L: int = 4096, H: int = 16, D: int = 128) -> Workload:
    """Linear chains: n_seq independent sequences of L tokens, random init states."""
    rng = np.random.default_rng(seed)
    T = n_seq * L
    parent = np.empty(T, dtype=np.int32)
    for s in range(n_seq):
        parent[s * L] = -1
        parent[s * L + 1:(s + 1) * L] = np.arange(s * L, (s + 1) * L - 1, dtype=np.int32)
    seq_start = (np.arange(n_seq + 1, dtype=np.int32) * L).astype(np.int32)
    q, k, v, beta, g = _values(rng, T, H, D, D, "bf16")
    init = _init(rng, n_seq, H, D, D, True)
    last = (seq_start[1:] - 1).astype(np.int32)
    return Workload(f"chains_{n_seq}x{L}_h{H}_d{D}", "bf16", parent, seq_start, q, k, v, beta, g,
                    init, None, last, info={"structure": f"{n_seq} chains x {L}"})


def decision_round(seed: int = 1002, n_req: int = 8, trunk: int = 8192, n_branch: int = 16, blen: int = 32,
            H: int = 16, D: int = 128) -> Workload:
    """Decision round: n_req requests, each a trunk with n_branch question
    branches of blen tokens forking from the trunk's final token. Readout rows
    and state rows are every branch's last token."""
    rng = np.random.default_rng(seed)
    per = trunk + n_branch * blen
    T = n_req * per
    parent = np.empty(T, dtype=np.int32)
    ends = []
    for r in range(n_req):
        a = r * per
        parent[a] = -1
        parent[a + 1:a + trunk] = np.arange(a, a + trunk - 1, dtype=np.int32)
        for b in range(n_branch):
            s = a + trunk + b * blen
            parent[s] = a + trunk - 1
            parent[s + 1:s + blen] = np.arange(s, s + blen - 1, dtype=np.int32)
            ends.append(s + blen - 1)
    seq_start = (np.arange(n_req + 1, dtype=np.int32) * per).astype(np.int32)
    q, k, v, beta, g = _values(rng, T, H, D, D, "bf16")
    init = _init(rng, n_req, H, D, D, False)
    ends = np.array(ends, dtype=np.int32)
    return Workload(f"decision_round_{n_req}x({trunk}+{n_branch}x{blen})_h{H}_d{D}", "bf16", parent,
                    seq_start, q, k, v, beta, g, init, ends.copy(), ends.copy(),
                    info={"structure": f"{n_req} x (trunk {trunk} + {n_branch} x {blen})"})


def random_draft_tree(rng, n_nodes: int = 64, max_depth: int = 8, max_fanout: int = 8) -> np.ndarray:
    """Random recursive tree laid out in DFS pre-order, children in creation
    order. Node n attaches uniformly to the virtual root (if it has fewer than
    max_fanout children) or to any node of depth < max_depth with fewer than
    max_fanout children. Returns local parents (-1 = child of the virtual root)."""
    par = []
    depth = []
    nchild = {-1: 0}
    for n in range(n_nodes):
        cand = []
        if nchild[-1] < max_fanout:
            cand.append(-1)
        cand += [u for u in range(n) if depth[u] < max_depth and nchild.get(u, 0) < max_fanout]
        p = cand[int(rng.integers(0, len(cand)))]
        par.append(p)
        depth.append(1 if p < 0 else depth[p] + 1)
        nchild[p] = nchild.get(p, 0) + 1
        nchild[n] = 0
    children = {u: [] for u in range(-1, n_nodes)}
    for n, p in enumerate(par):
        children[p].append(n)
    order = []
    stack = list(reversed(children[-1]))
    while stack:
        u = stack.pop()
        order.append(u)
        stack.extend(reversed(children[u]))
    newid = {u: i for i, u in enumerate(order)}
    out = np.empty(n_nodes, dtype=np.int32)
    for u in order:
        p = par[u]
        out[newid[u]] = -1 if p < 0 else newid[p]
    return out


def draft_trees(seed: int = 1003, n_seq: int = 64, n_nodes: int = 64, H: int = 32, D: int = 128) -> Workload:
    """Draft-tree verify: n_seq random trees of n_nodes over committed random
    states; all outputs and pseudo-values; then one root-to-leaf path per tree."""
    rng = np.random.default_rng(seed)
    T = n_seq * n_nodes
    parent = np.empty(T, dtype=np.int32)
    for s in range(n_seq):
        lp = random_draft_tree(rng, n_nodes)
        parent[s * n_nodes:(s + 1) * n_nodes] = np.where(lp < 0, -1, lp + s * n_nodes)
    seq_start = (np.arange(n_seq + 1, dtype=np.int32) * n_nodes).astype(np.int32)
    q, k, v, beta, g = _values(rng, T, H, D, D, "bf16")
    init = _init(rng, n_seq, H, D, D, True)
    lv = leaves_of(parent)
    ptr = [0]
    nodes = []
    for s in range(n_seq):
        mine = lv[(lv >= seq_start[s]) & (lv < seq_start[s + 1])]
        leaf = int(mine[int(rng.integers(0, mine.shape[0]))])
        path = root_path(parent, leaf)
        nodes += path
        ptr.append(len(nodes))
    wl = Workload(f"draft_trees_{n_seq}x{n_nodes}_h{H}_d{D}", "bf16", parent, seq_start, q, k, v, beta, g,
                  init, None, np.zeros(0, dtype=np.int32), keep_pseudo=True,
                  path_ptr=np.array(ptr, dtype=np.int32), path_nodes=np.array(nodes, dtype=np.int32),
                  path_seq=np.arange(n_seq, dtype=np.int32),
                  info={"structure": f"{n_seq} draft trees x {n_nodes} nodes"})
    return wl


def random_forest_tokens(rng, trunk_range=(512, 4096), branch_count=(1, 64), branch_len=(4, 256),
                         max_nest: int = 3):
    """One trunk with branches: each branch forks from a uniformly chosen
    existing token of nesting depth < max_nest. Laid out trunk first, then the
    branches in creation order. Returns local parents and nesting depths."""
    L = int(rng.integers(trunk_range[0], trunk_range[1] + 1))
    nb = int(rng.integers(branch_count[0], branch_count[1] + 1))
    par = [-1] + list(range(L - 1))
    nest = [0] * L
    for _ in range(nb):
        bl = int(rng.integers(branch_len[0], branch_len[1] + 1))
        elig = np.nonzero(np.array(nest) < max_nest)[0]
        fp = int(elig[int(rng.integers(0, elig.shape[0]))])
        d = nest[fp] + 1
        start = len(par)
        par.append(fp)
        nest.append(d)
        for i in range(1, bl):
            par.append(start + i - 1)
            nest.append(d)
    return np.array(par, dtype=np.int32), np.array(nest, dtype=np.int32)


def mixed_forest(seed: int = 1004, total: int = 65536, H: int = 32, D: int = 128, all_leaf_states: bool = False,
            **forest_kw) -> Workload:
    """Large mixed stream: seeded random forests (one trunk each, one sequence
    each) appended while they fit; the next one is cut in stream order to reach
    exactly `total` tokens."""
    rng = np.random.default_rng(seed)
    parents = []
    starts = [0]
    used = 0
    nests = []
    while used < total:
        lp, nest = random_forest_tokens(rng, **forest_kw)
        take = min(lp.shape[0], total - used)
        lp, nest = lp[:take], nest[:take]
        parents.append(np.where(lp < 0, -1, lp + used).astype(np.int32))
        nests.append(nest)
        used += take
        starts.append(used)
    parent = np.concatenate(parents).astype(np.int32)
    seq_start = np.array(starts, dtype=np.int32)
    n_seq = seq_start.shape[0] - 1
    T = parent.shape[0]
    q, k, v, beta, g = _values(rng, T, H, D, D, "bf16")
    init = _init(rng, n_seq, H, D, D, False)
    lv = leaves_of(parent)
    nest = np.concatenate(nests)
    n_branch = int(np.sum((parent >= 0) & (parent != np.arange(T) - 1)))
    return Workload(f"mixed_forest_{T}_h{H}_d{D}", "bf16", parent, seq_start, q, k, v, beta, g, init,
                    None, lv if all_leaf_states else np.zeros(0, dtype=np.int32),
                    info={"structure": f"{n_seq} forests, {n_branch} branches, {lv.shape[0]} leaves",
                          "n_forests": n_seq, "n_branches": n_branch, "n_leaves": int(lv.shape[0]),
                          "max_nest": int(nest.max())})


def random_small(seed: int, n_seq: int = 3, H: int = 2, Dk: int = 32, Dv: int = 32, dtype: str = "f32",
                 max_len: int = 200, random_init: bool = True) -> Workload:
    """Fuzz workload: a mix of chains, draft trees (<= 64 tokens) and forests
    with nested branches, small enough for the oracle in well under a second."""
    rng = np.random.default_rng(seed)
    parents = []
    starts = [0]
    used = 0
    for s in range(n_seq):
        kind = int(rng.integers(0, 3))
        if kind == 0:
            L = int(rng.integers(1, max_len + 1))
            lp = np.arange(-1, L - 1, dtype=np.int32)
        elif kind == 1:
            n = int(rng.integers(1, 65))
            lp = random_draft_tree(rng, n)
        else:
            lp, _ = random_forest_tokens(rng, trunk_range=(1, max(1, max_len // 2)), branch_count=(0, 6),
                                         branch_len=(1, 40))
        parents.append(np.where(lp < 0, -1, lp + used).astype(np.int32))
        used += lp.shape[0]
        starts.append(used)
    parent = np.concatenate(parents).astype(np.int32)
    seq_start = np.array(starts, dtype=np.int32)
    T = parent.shape[0]
    q, k, v, beta, g = _values(rng, T, H, Dk, Dv, dtype)
    init = _init(rng, n_seq, H, Dv, Dk, random_init)
    return Workload(f"random_small_{seed}", dtype, parent, seq_start, q, k, v, beta, g, init, None,
                    leaves_of(parent))


WORKLOADS = {"tiny_tree": tiny_tree, "chains": chains, "decision_round": decision_round, "draft_trees": draft_trees,
             "mixed_forest": mixed_forest}


def get(name: str, **kw) -> Workload:
    """A named workload at its default (full) size, or with sizes overridden."""
    return WORKLOADS[name](**kw)
