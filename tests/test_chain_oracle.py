"""Pins of the speculative chain-round reference (oracle/chain.py) against the
pinned per-token parent walk (oracle/gdn_oracle.c, TreeWY Eq. 1) and closed
forms: fully accepted rounds equal one chain over the concatenated drafts;
nothing accepted leaves the state unchanged; the committed state is the replay
of exactly the accepted tokens (Eq. 3's result); beta = 0 is pure decay."""
import numpy as np

import oracle
from oracle.chain import chain_rounds, chain_verify
from tree_forked_gated_amd import workloads as W


def _rounds(rng, n_seq, R, N, H, D):
    out = []
    for _ in range(R):
        q, k, v, beta, g = W._values(rng, n_seq * N, H, D, D, "f32")
        sh = lambda a: a.reshape((n_seq, N) + a.shape[1:])
        out.append({"q": sh(q), "k": sh(k), "v": sh(v), "beta": sh(beta), "log_gate": sh(g)})
    return out


def _chain_workload(S0, parts):
    """One chain per sequence over the concatenated draft tokens `parts`."""
    n_seq = S0.shape[0]
    cat = {f: np.concatenate([p[f] for p in parts], axis=1) for f in ("q", "k", "v", "beta", "log_gate")}
    L = cat["q"].shape[1]
    flat = lambda a: a.reshape((n_seq * L,) + a.shape[2:])
    parent = np.concatenate([np.arange(-1, L - 1) + (s * L if s else 0) * (np.arange(-1, L - 1) >= 0)
                             for s in range(n_seq)]).astype(np.int32)
    parent = np.where(parent < 0, -1, parent).astype(np.int32)
    seq_start = (np.arange(n_seq + 1) * L).astype(np.int32)
    return W.Workload("chain", "f32", parent, seq_start, flat(cat["q"]), flat(cat["k"]), flat(cat["v"]),
                      flat(cat["beta"]), flat(cat["log_gate"]), S0.astype(np.float32), None,
                      (seq_start[1:] - 1).astype(np.int32))


def test_fully_accepted_rounds_equal_one_chain():
    rng = np.random.default_rng(1)
    n_seq, R, N, H, D = 3, 5, 4, 2, 16
    S0 = W._init(rng, n_seq, H, D, D, True)
    rounds = _rounds(rng, n_seq, R, N, H, D)
    res, S = chain_rounds(S0, rounds, [np.full(n_seq, N)] * R)
    wl = _chain_workload(S0, rounds)
    ref = oracle.forward(wl, "f64")
    L = R * N
    out = ref["out"].reshape(n_seq, L, H, D)
    pv = ref["pseudo_v"].reshape(n_seq, L, H, D)
    for r in range(R):
        assert np.max(np.abs(res[r]["out"] - out[:, r * N:(r + 1) * N])) < 1e-12
        assert np.max(np.abs(res[r]["pseudo_v"] - pv[:, r * N:(r + 1) * N])) < 1e-12
    assert np.max(np.abs(S - ref["state"])) < 1e-12


def test_nothing_accepted_keeps_the_state():
    rng = np.random.default_rng(2)
    n_seq, R, N, H, D = 2, 4, 3, 2, 16
    S0 = W._init(rng, n_seq, H, D, D, True)
    rounds = _rounds(rng, n_seq, R, N, H, D)
    res, S = chain_rounds(S0, rounds, [np.zeros(n_seq, int)] * R)
    assert np.array_equal(S, S0.astype(np.float64))
    for r in range(R):
        assert np.array_equal(res[r]["start_state"], S0.astype(np.float64))
        wl = _chain_workload(S0, [rounds[r]])
        ref = oracle.forward(wl, "f64")
        assert np.max(np.abs(res[r]["out"] - ref["out"].reshape(n_seq, N, H, D))) < 1e-12


def test_committed_state_is_the_replay_of_the_accepted_tokens():
    rng = np.random.default_rng(3)
    n_seq, R, N, H, D = 4, 6, 4, 2, 16
    S0 = W._init(rng, n_seq, H, D, D, True)
    rounds = _rounds(rng, n_seq, R, N, H, D)
    acc = [rng.integers(0, N + 1, n_seq) for _ in range(R)]
    _, S = chain_rounds(S0, rounds, acc)
    for s in range(n_seq):
        # the accepted tokens of every round, concatenated, replayed as one chain from S0
        kept = [{f: rounds[r][f][s:s + 1, :acc[r][s]] for f in rounds[r]} for r in range(R)]
        wl = _chain_workload(S0[s:s + 1], kept)
        if wl.T == 0:
            assert np.array_equal(S[s], S0[s])
            continue
        ref = oracle.forward(wl, "f64")
        assert np.max(np.abs(S[s] - ref["state"][0])) < 1e-12


def test_beta_zero_is_pure_decay():
    rng = np.random.default_rng(4)
    H, D, N = 2, 8, 5
    S0 = rng.standard_normal((H, D, D))
    q, k, v, _, g = W._values(rng, N, H, D, D, "f32")
    out, pv, st = chain_verify(S0, q, k, v, np.zeros((N, H)), g)
    G = np.cumsum(g.astype(np.float64), axis=0)
    for t in range(N):
        for h in range(H):
            assert np.max(np.abs(st[t, h] - np.exp(G[t, h]) * S0[h])) < 1e-12
            assert np.max(np.abs(out[t, h] - np.exp(G[t, h]) * S0[h] @ q[t, h])) < 1e-12
    assert np.array_equal(pv, np.zeros_like(pv))
