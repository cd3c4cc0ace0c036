"""Reference speculative chain rounds — TEST INFRASTRUCTURE ONLY.

Only tests/, __graft_entry__.smoke() and bench.py's CPU-baseline leg use this
module; the library never imports it.

What it computes (TreeWY, "Speculative Verification for Gated DeltaNet
Hybrids", section 4 "Implementation": a chain draft verifies and commits in one
kernel; appendix D and the ReplaySSM paragraph of section 1: the committed
state is materialised only at a periodic flush). A sequence decodes in rounds.
Round r starts from the committed state S_r and verifies a chain draft of N
tokens: every draft token's output and pseudo-value come from the per-token
recurrence (TreeWY section 1, Eq. 1, with the key rewrite of section 3)

    vt_t = beta_t (v_t - alpha_t S_{t-1} k_t),   S_t = alpha_t S_{t-1} + vt_t k_t^T,   o_t = S_t q_t

starting at S_r. The caller then accepts the first a_r draft tokens, and the
next round starts from S_{r+1}, the state after them (S_r when a_r = 0). When
and where S_{r+1} is written to memory (every round, or at a flush with the
accepted tokens kept as history until then) does not change any value, so the
reference keeps S_r exactly, in fp64, by plain replay.
"""
from __future__ import annotations

import numpy as np


def chain_verify(S0: np.ndarray, q, k, v, beta, log_gate):
    """Per-token recurrence of one chain draft from S0 ([H, Dv, Dk]).
    q, k [N, H, Dk], v [N, H, Dv], beta, log_gate [N, H]. Returns (out
    [N, H, Dv], pseudo_v [N, H, Dv], states [N, H, Dv, Dk] after each token)."""
    S = np.array(S0, dtype=np.float64)
    N, H = q.shape[0], q.shape[1]
    Dv = v.shape[2]
    out = np.zeros((N, H, Dv))
    pv = np.zeros((N, H, Dv))
    states = np.zeros((N,) + S.shape)
    for t in range(N):
        for h in range(H):
            a = np.exp(np.float64(log_gate[t, h]))
            kt = np.asarray(k[t, h], np.float64)
            u = S[h] @ kt
            vt = np.float64(beta[t, h]) * (np.asarray(v[t, h], np.float64) - a * u)
            S[h] = a * S[h] + np.outer(vt, kt)
            out[t, h] = S[h] @ np.asarray(q[t, h], np.float64)
            pv[t, h] = vt
        states[t] = S
    return out, pv, states


def chain_rounds(S0: np.ndarray, rounds, accepted):
    """S0 [n_seq, H, Dv, Dk]; rounds: list of dicts with q, k, v, beta,
    log_gate of shape [n_seq, N, H, D] (or [n_seq, N, H]); accepted: list of
    int arrays [n_seq] (draft tokens accepted after each round, 0..N).
    Returns, per round, the outputs and pseudo-values of the draft and the
    committed state it started from, plus the state after the last round's
    accepted tokens."""
    S = np.array(S0, dtype=np.float64)
    res = []
    for rd, acc in zip(rounds, accepted):
        n_seq = S.shape[0]
        outs, pvs, starts = [], [], S.copy()
        nxt = S.copy()
        for s in range(n_seq):
            o, pv, st = chain_verify(S[s], rd["q"][s], rd["k"][s], rd["v"][s], rd["beta"][s], rd["log_gate"][s])
            outs.append(o)
            pvs.append(pv)
            a = int(acc[s])
            if not 0 <= a <= o.shape[0]:
                raise ValueError(f"accepted count {a} outside [0, {o.shape[0]}]")
            if a > 0:
                nxt[s] = st[a - 1]
        res.append({"out": np.stack(outs), "pseudo_v": np.stack(pvs), "start_state": starts})
        S = nxt
    return res, S
