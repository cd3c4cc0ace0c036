"""Reference tree metadata — TEST INFRASTRUCTURE ONLY.

The GPU builds the tree's metadata itself (Flide, "Accelerating Decision
Inference with Exact State Forking", section 3.3.1: everything that depends on
the round's composition lives in device buffers the kernels read). This module
computes the same tables with plain loops, from these definitions:

* validation: seq_start is a CSR over [0, T]; every parent is -1 or a token of
  the same sequence with a smaller index (TreeWY, "Speculative Verification
  for Gated DeltaNet Hybrids", section 3 "Verifying a draft": parents precede
  children). The error word is the smallest (code, index) found.
* depth: 0 for a token whose parent is -1, else parent's depth + 1.
* execution mode: a sequence of at most 64 tokens is one tree chunk (its
  whole draft tree solved at once, TreeWY Eq. 2) with a 64 x 64 ancestor-or-self
  bit mask; a longer sequence is cut into segments, each starting at a token
  whose parent is not the token just before it (a root or a fork), and each
  segment into chunks of 64 tokens counted from its start (Flide section 3.5:
  chunks of a question start exactly at its fork).
* fork slots: every token that a segment start of a long sequence names as
  parent gets a slot, numbered in stream order; the segment's entry state is
  that slot.
* level: 0 for a segment whose entry is an initial state, else the level of
  the segment holding its entry token plus one.
* rows: out_rows and state_rows must be distinct tokens in [0, T).
"""
from __future__ import annotations

import numpy as np

CHUNK = 64

DEV_OK = 0
DEV_SEQ_START = 1
DEV_PARENT_ORDER = 2
DEV_PARENT_SEQ = 3
DEV_FORK_CAPACITY = 4
DEV_LEVEL_CAPACITY = 5
DEV_ROWS = 6
DEV_PATH = 7


def plan(parent, seq_start, max_forks=None, max_levels=None, out_rows=None, state_rows=None):
    parent = [int(x) for x in np.asarray(parent)]
    seq_start = [int(x) for x in np.asarray(seq_start)]
    T = len(parent)
    n_seq = len(seq_start) - 1
    errs = []

    def err(code, idx):
        errs.append((code, idx))

    # seq_start
    if n_seq < 0 or seq_start[0] != 0:
        err(DEV_SEQ_START, 0)
    for s in range(n_seq):
        if seq_start[s + 1] < seq_start[s] or seq_start[s + 1] > T:
            err(DEV_SEQ_START, s + 1)
    if n_seq >= 0 and seq_start[n_seq] != T:
        err(DEV_SEQ_START, n_seq)
    if errs:
        return {"error": min(errs)}

    tok_seq = [0] * T
    for s in range(n_seq):
        for t in range(seq_start[s], seq_start[s + 1]):
            tok_seq[t] = s
    for t in range(T):
        p = parent[t]
        if p < -1 or p >= t:
            err(DEV_PARENT_ORDER, t)
        elif p >= 0 and p < seq_start[tok_seq[t]]:
            err(DEV_PARENT_SEQ, t)
    if errs:
        return {"error": min(errs)}

    depth = [0] * T
    for t in range(T):
        depth[t] = 0 if parent[t] < 0 else depth[parent[t]] + 1

    tree_seq = [(seq_start[s + 1] - seq_start[s]) <= CHUNK for s in range(n_seq)]
    is_start = [False] * T
    for t in range(T):
        s = tok_seq[t]
        if tree_seq[s]:
            is_start[t] = (t == seq_start[s])
        else:
            is_start[t] = parent[t] < 0 or parent[t] != t - 1

    starts = [t for t in range(T) if is_start[t]]
    n_seg = len(starts)
    seg_of = [0] * T
    cur = -1
    for t in range(T):
        if is_start[t]:
            cur += 1
        seg_of[t] = cur
    seg_len = [(starts[i + 1] if i + 1 < n_seg else T) - starts[i] for i in range(n_seg)]
    seg_seq = [tok_seq[a] for a in starts]
    seg_mode = [1 if tree_seq[tok_seq[a]] else 0 for a in starts]
    seg_entry = [(-1 if seg_mode[i] else parent[a]) for i, a in enumerate(starts)]

    is_fork = [False] * T
    for e in seg_entry:
        if e >= 0:
            is_fork[e] = True
    fork_slot = [-1] * T
    n_fork = 0
    for t in range(T):
        if is_fork[t]:
            fork_slot[t] = n_fork
            n_fork += 1
    seg_slot = [(fork_slot[e] if e >= 0 else -1) for e in seg_entry]

    seg_level = [0] * n_seg
    for i in range(n_seg):
        e = seg_entry[i]
        seg_level[i] = 0 if e < 0 else seg_level[seg_of[e]] + 1

    masks = np.zeros((n_seq, CHUNK), dtype=np.uint64)
    for s in range(n_seq):
        if not tree_seq[s]:
            continue
        a = seq_start[s]
        for t in range(a, seq_start[s + 1]):
            m = 0
            u = t
            while u >= 0:
                m |= 1 << (u - a)
                u = parent[u]
            masks[s, t - a] = np.uint64(m)

    if max_forks is not None and n_fork > max_forks:
        first_over = [t for t in range(T) if fork_slot[t] == max_forks][0]
        err(DEV_FORK_CAPACITY, first_over)
    if max_levels is not None:
        for i in range(n_seg):
            if seg_level[i] >= max_levels:
                err(DEV_LEVEL_CAPACITY, starts[i])

    def rows_check(rows):
        if rows is None:
            return
        seen = {}
        for i, r in enumerate(int(x) for x in np.asarray(rows)):
            if r < 0 or r >= T or r in seen:
                err(DEV_ROWS, i)
            else:
                seen[r] = i

    rows_check(out_rows)
    rows_check(state_rows)

    n_chunks = [1 if seg_mode[i] else -(-seg_len[i] // CHUNK) for i in range(n_seg)]
    return {
        "error": min(errs) if errs else (DEV_OK, 0),
        "tok_seq": np.array(tok_seq, dtype=np.int32),
        "depth": np.array(depth, dtype=np.int32),
        "fork_slot": np.array(fork_slot, dtype=np.int32),
        "n_fork": n_fork,
        "seg_start": np.array(starts, dtype=np.int32),
        "seg_len": np.array(seg_len, dtype=np.int32),
        "seg_seq": np.array(seg_seq, dtype=np.int32),
        "seg_mode": np.array(seg_mode, dtype=np.int32),
        "seg_entry": np.array(seg_entry, dtype=np.int32),
        "seg_slot": np.array(seg_slot, dtype=np.int32),
        "seg_level": np.array(seg_level, dtype=np.int32),
        "seg_nchunks": np.array(n_chunks, dtype=np.int32),
        "n_seg": n_seg,
        "n_levels": (max(seg_level) + 1) if n_seg else 0,
        "tree_mask": masks,
    }
