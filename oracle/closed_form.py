"""TreeWY closed form, dense fp64, for tiny trees — TEST INFRASTRUCTURE ONLY.

TreeWY ("Speculative Verification for Gated DeltaNet Hybrids"), section 3:

* "Verifying a draft", Eq. 2: with the nodes in an order where parents come
  first, all pseudo-values solve one system
      (I + diag(beta) G) Vt = R,
      G[t, i] = (g_t / g_i) (k_t . k_i)   for i a strict ancestor of t, else 0,
      R[t]    = beta_t v_t - beta_t g_t (S_0 k_t),
  where g_t is the product of the decays alpha on the root path of t,
  t included. (The page lost the fraction bar of g_t / g_i; the quotient is
  the reading that satisfies Eq. 1.)
* "Reconstruct on commit", Eq. 3: the state after node a is
      S_a = g_a S_0 + sum over i ancestor-or-self of a of (g_a / g_i) vt_i k_i^T,
  and the output of node a is o_a = S_a q_a.

This is a second, independent route to the oracle's result: no state is ever
walked from token to token. g_a / g_i is evaluated as exp(G_a - G_i) with G the
path sum of log gates, which is the same number without underflow.
"""
from __future__ import annotations

import numpy as np
from scipy.linalg import solve_triangular


def ancestor_matrix(parent_local: np.ndarray) -> np.ndarray:
    """anc[t, i] = True iff i is an ancestor of t or t itself (walks parents)."""
    n = parent_local.shape[0]
    anc = np.zeros((n, n), dtype=bool)
    for t in range(n):
        u = t
        while u >= 0:
            anc[t, u] = True
            u = int(parent_local[u])
    return anc


def path_log_decay(parent_local: np.ndarray, log_gate: np.ndarray) -> np.ndarray:
    """G[t] = sum of log gates over the root path of t, t included (fp64)."""
    n = parent_local.shape[0]
    G = np.zeros(n, dtype=np.float64)
    for t in range(n):
        p = int(parent_local[t])
        G[t] = np.float64(log_gate[t]) + (G[p] if p >= 0 else 0.0)
    return G


def tree_wy(parent_local, q, k, v, beta, log_gate, S0):
    """One sequence, one head. Shapes: q,k [n,Dk], v [n,Dv], beta/log_gate [n],
    S0 [Dv,Dk]. Returns (out [n,Dv], pseudo [n,Dv], states [n,Dv,Dk]) in fp64."""
    q, k, v = (np.asarray(a, dtype=np.float64) for a in (q, k, v))
    beta = np.asarray(beta, dtype=np.float64)
    S0 = np.asarray(S0, dtype=np.float64)
    n = parent_local.shape[0]
    anc = ancestor_matrix(parent_local)
    strict = anc & ~np.eye(n, dtype=bool)
    G = path_log_decay(parent_local, log_gate)
    ratio = np.exp(np.where(anc, G[:, None] - G[None, :], -np.inf))  # g_t / g_i on ancestors, 0 elsewhere
    Gm = np.where(strict, ratio * (k @ k.T), 0.0)
    M = np.eye(n) + beta[:, None] * Gm
    R = beta[:, None] * v - (beta * np.exp(G))[:, None] * (k @ S0.T)
    pseudo = solve_triangular(M, R, lower=True)
    states = np.exp(G)[:, None, None] * S0[None] + np.einsum("ai,iv,id->avd", ratio, pseudo, k)
    out = np.einsum("avd,ad->av", states, q)
    return out, pseudo, states


def commit_state(path_local, q_unused, k, pseudo, log_gate, S0):
    """Eq. 3 along one root-to-node path given its pseudo-values (fp64)."""
    k = np.asarray(k, dtype=np.float64)
    pseudo = np.asarray(pseudo, dtype=np.float64)
    G = np.cumsum(np.asarray(log_gate, dtype=np.float64)[path_local])
    if len(path_local) == 0:
        return np.asarray(S0, dtype=np.float64).copy()
    Ga = G[-1]
    S = np.exp(Ga) * np.asarray(S0, dtype=np.float64)
    for j, t in enumerate(path_local):
        S = S + np.exp(Ga - G[j]) * np.outer(pseudo[t], k[t])
    return S
