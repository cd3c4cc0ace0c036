"""Reference ForkAttention for full-attention layers — TEST INFRASTRUCTURE ONLY.

Only tests/, __graft_entry__.smoke() and bench.py's CPU-baseline leg use this
module; the library never imports it.

What it computes (Flide, "Accelerating Decision Inference with Exact State
Forking", section 3.2.1 "Full-Attention Layers"; the visibility rule, the
page's Equation 3, did not survive extraction). Reading: a token attends to the
tokens on its own root path, itself included, in its own sequence, i.e. its
ancestors-or-self along parent pointers. This is the rule under which, in a
causal model where the shared state never attends to a question, every question
computes exactly its standalone prompt s (+) q_i (section 3.2.3, the exactness
statement), and under which no request sees another request's tokens (section
3.3.1: the kernel skips the states of other requests). With a chain it is
ordinary causal attention.

For query head h (with Hq = G Hkv query heads grouped over Hkv key/value
heads, key/value head h // G):

    o_t = sum over j ancestor-or-self of t of softmax_j(scale * q_t . k_j) v_j

plain per token, in fp64, walking the parent pointers. Small inputs only.

Cached keys (section 3.4, incremental state forking: a checkpoint keeps the
keys and values of the full-attention layers before its position, and a
resumed request's tokens come after them). Sequence s may have cached rows
[cache_start[s], cache_start[s + 1]) of k_cache and v_cache: they precede the
sequence's roots, so every token of s sees all of them, before its root path.
"""
from __future__ import annotations

import numpy as np


def visible_tokens(parent: np.ndarray, t: int) -> np.ndarray:
    """Ancestors-or-self of token t, from the root down."""
    path = []
    while t >= 0:
        path.append(t)
        t = int(parent[t])
    return np.array(path[::-1], dtype=np.int64)


def check_structure(parent: np.ndarray, seq_start: np.ndarray) -> None:
    """Parents precede their children inside the same sequence (as for the
    recurrence); raises ValueError otherwise."""
    T = parent.shape[0]
    if seq_start[0] != 0 or seq_start[-1] != T or np.any(np.diff(seq_start) < 0):
        raise ValueError("seq_start is not a CSR over [0, T]")
    for s in range(seq_start.shape[0] - 1):
        a, b = int(seq_start[s]), int(seq_start[s + 1])
        for t in range(a, b):
            p = int(parent[t])
            if p != -1 and not (a <= p < t):
                raise ValueError(f"token {t}: parent {p} is not an earlier token of its sequence")


def fork_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, parent: np.ndarray, seq_start: np.ndarray,
                   scale: float, rows=None, k_cache=None, v_cache=None, cache_start=None) -> np.ndarray:
    """Outputs [len(rows) or T, Hq, D] in fp64 for q [T, Hq, D], k and v
    [T, Hkv, D]. rows: the tokens to compute (default: all), one by one.
    k_cache, v_cache [Tc, Hkv, D] and cache_start [n_seq + 1]: optional
    cached keys and values of each sequence."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    parent = np.asarray(parent, np.int64)
    seq_start = np.asarray(seq_start, np.int64)
    check_structure(parent, seq_start)
    if cache_start is not None:
        cache_start = np.asarray(cache_start, np.int64)
        k_cache = np.asarray(k_cache, np.float64)
        v_cache = np.asarray(v_cache, np.float64)
        if cache_start.shape != seq_start.shape or cache_start[0] != 0 or np.any(np.diff(cache_start) < 0) \
                or cache_start[-1] != k_cache.shape[0]:
            raise ValueError("cache_start is not a CSR over the cached rows, one range per sequence")
    tok_seq = np.searchsorted(seq_start, np.arange(parent.shape[0]), side="right") - 1
    T, Hq, D = q.shape
    Hkv = k.shape[1]
    if Hq % Hkv:
        raise ValueError("query heads must be a multiple of key/value heads")
    G = Hq // Hkv
    rows = np.arange(T) if rows is None else np.asarray(rows, np.int64)
    out = np.zeros((rows.shape[0], Hq, D))
    for i, t in enumerate(rows):
        vis = visible_tokens(parent, int(t))
        for h in range(Hq):
            g = h // G
            keys, vals = k[vis, g, :], v[vis, g, :]
            if cache_start is not None:
                s = tok_seq[t]
                c = slice(cache_start[s], cache_start[s + 1])
                keys = np.concatenate([k_cache[c, g, :], keys])
                vals = np.concatenate([v_cache[c, g, :], vals])
            logits = scale * (keys @ q[t, h, :])
            w = np.exp(logits - logits.max())
            out[i, h] = (w / w.sum()) @ vals
    return out
