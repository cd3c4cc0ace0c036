"""Pins of the ForkAttention oracle (oracle/attention.py) against facts that do
not come from it: textbook causal attention (torch's scaled_dot_product_attention
on the CPU in float64), the standalone-prompt exactness statement of Flide
("Accelerating Decision Inference with Exact State Forking", section 3.2.3),
closed forms, and a dense masked softmax whose mask is the transitive closure
of the parent relation (boolean matrix products, not a pointer walk)."""
import numpy as np
import pytest
import torch

from oracle.attention import fork_attention, visible_tokens


def _qkv(rng, T, Hq, Hkv, D):
    q = rng.standard_normal((T, Hq, D))
    k = rng.standard_normal((T, Hkv, D))
    v = rng.standard_normal((T, Hkv, D))
    return q, k, v


def _causal_sdpa(q, k, v, scale):
    """Textbook causal attention over one sequence ([n, H, D], same heads)."""
    tq = torch.from_numpy(q).permute(1, 0, 2)[None]
    tk = torch.from_numpy(k).permute(1, 0, 2)[None]
    tv = torch.from_numpy(v).permute(1, 0, 2)[None]
    o = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=True, scale=scale)
    return o[0].permute(1, 0, 2).numpy()


def _forest():
    """Trunk of 40 tokens, branches off tokens 39, 17 and 0, one nested in the
    second branch; local parents."""
    par = list(range(-1, 39))
    spans = []
    for ft, bl in [(39, 6), (17, 9), (0, 3)]:
        b0 = len(par)
        par += [ft] + list(range(b0, b0 + bl - 1))
        spans.append((b0, len(par)))
    b0 = len(par)
    par += [spans[1][0] + 4] + list(range(b0, b0 + 4))  # nested: off the 5th token of the second branch
    spans.append((b0, len(par)))
    return np.array(par, np.int64), spans


def test_chain_is_causal_attention():
    rng = np.random.default_rng(1)
    T, H, D = 50, 3, 16
    q, k, v = _qkv(rng, T, H, H, D)
    par = np.arange(-1, T - 1)
    got = fork_attention(q, k, v, par, np.array([0, T]), 0.3)
    ref = _causal_sdpa(q, k, v, 0.3)
    assert np.max(np.abs(got - ref)) < 1e-12


def test_every_token_computes_its_standalone_prompt():
    """Section 3.2.3: a question token's output equals the one it gets when its
    root path (the shared state up to the fork, then the question) is processed
    alone as one causal sequence."""
    rng = np.random.default_rng(2)
    par, spans = _forest()
    T, H, D = par.shape[0], 2, 8
    q, k, v = _qkv(rng, T, H, H, D)
    got = fork_attention(q, k, v, par, np.array([0, T]), 0.5)
    for t in range(T):
        path = visible_tokens(par, t)
        ref = _causal_sdpa(q[path], k[path], v[path], 0.5)[-1]
        assert np.max(np.abs(got[t] - ref)) < 1e-12, t


def test_no_sibling_leak_and_negative_control():
    rng = np.random.default_rng(3)
    par, spans = _forest()
    T, H, D = par.shape[0], 2, 8
    q, k, v = _qkv(rng, T, H, H, D)
    seq = np.array([0, T])
    base = fork_attention(q, k, v, par, seq, 0.5)
    b = spans[0]  # the first branch; perturb the other branches' tokens
    others = np.r_[spans[1][0]:spans[1][1], spans[2][0]:spans[2][1], spans[3][0]:spans[3][1]]
    k2, v2 = k.copy(), v.copy()
    k2[others] += 1.0
    v2[others] -= 2.0
    pert = fork_attention(q, k2, v2, par, seq, 0.5)
    assert np.array_equal(base[b[0]:b[1]], pert[b[0]:b[1]])
    # negative control: the same tokens laid out as one chain (a delimiter-style
    # concatenation) do see the perturbed tokens before them
    chain = np.arange(-1, T - 1)
    last = spans[3][1] - 1
    c0 = fork_attention(q, k, v, chain, seq, 0.5, rows=[last])
    c1 = fork_attention(q, k2, v2, chain, seq, 0.5, rows=[last])
    assert np.max(np.abs(c0 - c1)) > 1e-3


def test_closed_forms():
    rng = np.random.default_rng(4)
    par, _ = _forest()
    T, H, D = par.shape[0], 2, 8
    q, k, v = _qkv(rng, T, H, H, D)
    seq = np.array([0, T])
    # a root sees only itself: its output is its value
    got = fork_attention(q, k, v, par, seq, 0.5, rows=[0])
    assert np.array_equal(got[0], v[0])
    # equal keys: uniform weights over the root path, i.e. the mean of its values
    kc = np.broadcast_to(k[:1], k.shape).copy()
    got = fork_attention(q, kc, v, par, seq, 0.5)
    for t in [5, 39, 45, T - 1]:
        path = visible_tokens(par, t)
        assert np.max(np.abs(got[t] - v[path].mean(axis=0))) < 1e-12


def test_dense_mask_from_transitive_closure():
    """The same outputs from one masked softmax per head whose mask is the
    reflexive-transitive closure of 'parent of' (boolean matrix squaring)."""
    rng = np.random.default_rng(5)
    par, _ = _forest()
    T, H, D = par.shape[0], 3, 8
    q, k, v = _qkv(rng, T, H, H, D)
    A = np.zeros((T, T), bool)  # A[i, j]: j is the parent of i
    for i, p in enumerate(par):
        if p >= 0:
            A[i, p] = True
    M = A | np.eye(T, dtype=bool)
    for _ in range(7):  # paths of length up to 2^7 > T
        M = M | ((M.astype(np.int64) @ M.astype(np.int64)) > 0)
    got = fork_attention(q, k, v, par, np.array([0, T]), 0.7)
    for h in range(H):
        logits = 0.7 * q[:, h, :] @ k[:, h, :].T
        logits = np.where(M, logits, -np.inf)
        w = np.exp(logits - logits.max(axis=1, keepdims=True))
        ref = (w / w.sum(axis=1, keepdims=True)) @ v[:, h, :]
        assert np.max(np.abs(got[:, h] - ref)) < 1e-12


def test_grouped_heads_equal_repeated_keys_and_values():
    rng = np.random.default_rng(6)
    par, _ = _forest()
    T, Hq, Hkv, D = par.shape[0], 6, 2, 8
    q, k, v = _qkv(rng, T, Hq, Hkv, D)
    seq = np.array([0, T])
    got = fork_attention(q, k, v, par, seq, 0.4)
    rep = fork_attention(q, np.repeat(k, Hq // Hkv, axis=1), np.repeat(v, Hq // Hkv, axis=1), par, seq, 0.4)
    assert np.array_equal(got, rep)


def test_requests_are_isolated_and_structure_checked():
    rng = np.random.default_rng(7)
    par, _ = _forest()
    n = par.shape[0]
    T = 2 * n
    parent = np.concatenate([par, np.where(par < 0, -1, par + n)])
    q, k, v = _qkv(rng, T, 2, 2, 8)
    both = fork_attention(q, k, v, parent, np.array([0, n, T]), 0.5)
    alone = fork_attention(q[n:], k[n:], v[n:], par, np.array([0, n]), 0.5)
    assert np.array_equal(both[n:], alone)
    bad = parent.copy()
    bad[n + 3] = 2  # a parent in the other request
    with pytest.raises(ValueError):
        fork_attention(q, k, v, bad, np.array([0, n, T]), 0.5)


def test_cached_keys_act_as_the_sequence_prefix():
    """Section 3.4: a request resumed from a checkpoint with cached keys and
    values computes what the fresh request computes when the cached part is
    real tokens ahead of it (a chain prefix that every root hangs off)."""
    rng = np.random.default_rng(8)
    par, _ = _forest()
    n = par.shape[0]
    C, H, D = 23, 2, 8
    q, k, v = _qkv(rng, n + C, H, H, D)
    # fresh: C prefix tokens as a chain, the forest's roots hang off the last of them
    fresh_par = np.concatenate([np.arange(-1, C - 1), np.where(par < 0, C - 1, par + C)])
    fresh = fork_attention(q, k, v, fresh_par, np.array([0, n + C]), 0.6)
    # resumed: the prefix only as cached keys and values
    resumed = fork_attention(q[C:], k[C:], v[C:], par, np.array([0, n]), 0.6, k_cache=k[:C], v_cache=v[:C],
                             cache_start=np.array([0, C]))
    assert np.max(np.abs(resumed - fresh[C:])) < 1e-12


def test_caches_belong_to_their_sequence():
    rng = np.random.default_rng(9)
    par, _ = _forest()
    n = par.shape[0]
    T = 2 * n
    parent = np.concatenate([par, np.where(par < 0, -1, par + n)])
    q, k, v = _qkv(rng, T, 2, 2, 8)
    kc, vc = rng.standard_normal((30, 2, 8)), rng.standard_normal((30, 2, 8))
    both = fork_attention(q, k, v, parent, np.array([0, n, T]), 0.5, k_cache=kc, v_cache=vc,
                          cache_start=np.array([0, 0, 30]))  # only the second request has cached rows
    first = fork_attention(q[:n], k[:n], v[:n], par, np.array([0, n]), 0.5)
    second = fork_attention(q[n:], k[n:], v[n:], par, np.array([0, n]), 0.5, k_cache=kc, v_cache=vc,
                            cache_start=np.array([0, 30]))
    assert np.array_equal(both[:n], first) and np.array_equal(both[n:], second)
    with pytest.raises(ValueError):
        fork_attention(q, k, v, parent, np.array([0, n, T]), 0.5, k_cache=kc, v_cache=vc,
                       cache_start=np.array([0, 10, 20]))
