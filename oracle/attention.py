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
                   scale: float, rows=None) -> np.ndarray:
    """Outputs [len(rows) or T, Hq, D] in fp64 for q [T, Hq, D], k and v
    [T, Hkv, D]. rows: the tokens to compute (default: all), one by one."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    parent = np.asarray(parent, np.int64)
    check_structure(parent, np.asarray(seq_start, np.int64))
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
            logits = scale * (k[vis, g, :] @ q[t, h, :])
            w = np.exp(logits - logits.max())
            out[i, h] = (w / w.sum()) @ v[vis, g, :]
    return out
