"""Offsets past 2^31 elements.

A stream of 4,100 sequences of 128 tokens (524,800 tokens), 32 heads, d_k =
d_v = 128: q, k, v, the outputs, the pseudo-values, the initial states and the
fork-state slots each hold more than 2^31 elements, and the last sequences'
rows lie past 2^31 elements from the start of every one of them. Each sequence
is a 96-token trunk with a 32-token branch that forks from trunk token 40 (a
mid-chunk fork, two levels). Inputs are drawn on the device with torch's
seeded generator, following the synthetic workloads' recipe (q and k standard
normal and L2-normalised per token and head, v standard normal, beta =
sigmoid, log gate = -softplus of standard normals, initial states N(0, 0.02)),
then rounded to bf16.

Sequences are independent, so the oracle runs on six sampled sequences alone
(both ends of the stream and its middle), re-based to a stream of their own:
the forward's outputs and leaf states, the commit of each sampled sequence's
root-to-branch-leaf path, and ForkAttention with 32 query heads over 2
key/value heads. Tolerances as for the other bf16 streams: relative L2 1e-2,
and no row beyond 5e-2 of the typical row norm.
"""
import numpy as np
import pytest
import torch

import oracle
from oracle.attention import fork_attention
from tree_forked_gated_amd import workloads as W

from gpu_helpers import f64, record_margin, rel_l2, say

pytestmark = pytest.mark.gpu

N_SEQ, TRUNK, BR, FORK = 4100, 96, 32, 40
H, D = 32, 128
SAMPLE = [0, 1, 2050, 4097, 4098, 4099]
TOL, ROW_TOL = 1e-2, 5e-2


def _structure():
    L = TRUNK + BR
    local = np.array(list(range(-1, TRUNK - 1)) + [FORK] + list(range(TRUNK, TRUNK + BR - 1)), np.int64)
    base = np.arange(N_SEQ, dtype=np.int64)[:, None] * L
    parent = np.where(local[None, :] < 0, -1, local[None, :] + base).ravel().astype(np.int32)
    seq_start = (np.arange(N_SEQ + 1, dtype=np.int64) * L).astype(np.int32)
    return parent, seq_start


def _inputs(T):
    gen = torch.Generator(device="cuda")
    gen.manual_seed(4242)

    def normal(shape, unit=False):
        x = torch.randn(shape, generator=gen, device="cuda", dtype=torch.float32)
        return x / x.norm(dim=-1, keepdim=True) if unit else x

    q = normal((T, H, D), True).to(torch.bfloat16)
    k = normal((T, H, D), True).to(torch.bfloat16)
    v = normal((T, H, D)).to(torch.bfloat16)
    beta = torch.sigmoid(normal((T, H))).to(torch.bfloat16)
    log_gate = (-torch.nn.functional.softplus(normal((T, H)))).to(torch.bfloat16)
    init = normal((N_SEQ, H, D, D)) * 0.02
    return q, k, v, beta, log_gate, init


def _rows_worst(gpu, ref):
    axes = (-1,) if gpu.ndim == 3 else (-2, -1)
    err = np.sqrt(np.sum((gpu - ref) ** 2, axis=axes))
    return float(err.max() / max(np.sqrt(np.mean(np.sum(ref ** 2, axis=axes))), 1e-30))


def _sample(parent, seq_start, tensors, init):
    """The sampled sequences as a stream of their own: token indices in the big
    stream, re-based parents, their inputs on the host."""
    toks, par, starts = [], [], [0]
    for s in SAMPLE:
        a, b = int(seq_start[s]), int(seq_start[s + 1])
        p = parent[a:b].astype(np.int64)
        par.append(np.where(p < 0, -1, p - a + starts[-1]))
        toks.append(np.arange(a, b))
        starts.append(starts[-1] + (b - a))
    toks = np.concatenate(toks)
    idx = torch.from_numpy(toks).cuda()
    host = [t.index_select(0, idx).float().cpu().numpy() for t in tensors]
    ini = init.index_select(0, torch.tensor(SAMPLE, device="cuda")).cpu().numpy()
    return toks, np.concatenate(par).astype(np.int32), np.array(starts, np.int32), host, ini


def test_offsets_past_2_31_elements():
    from tree_forked_gated_amd import binding as B
    parent, seq_start = _structure()
    T = int(parent.shape[0])
    assert T * H * D > 2 ** 31 and N_SEQ * H * D * D > 2 ** 31
    q, k, v, beta, log_gate, init = _inputs(T)
    leaves = W.leaves_of(parent)
    sample_leaves = np.array([x for x in leaves if np.searchsorted(seq_start, x, side="right") - 1 in SAMPLE],
                             np.int32)
    say(f"large stream: T={T} H={H} d={D}, {N_SEQ} sequences; {T * H * D} elements per q/k/v")
    cap = B.capacities(parent, seq_start)
    pd = torch.from_numpy(parent).cuda()
    sd = torch.from_numpy(seq_start).cuda()
    res = B.forward(q, k, v, log_gate, beta, pd, sd, init, state_rows=sample_leaves, keep_pseudo=True,
                    max_forks=cap["max_forks"], max_levels=cap["max_levels"], check=True)
    torch.cuda.synchronize()

    toks, spar, sstart, (hq, hk, hv, hb, hg), hini = _sample(parent, seq_start, (q, k, v, beta, log_gate), init)
    sleaves = W.leaves_of(spar)
    wl = W.Workload("large_sample", "bf16", spar, sstart, hq, hk, hv, hb, hg, hini, None, sleaves)
    ref = oracle.forward(wl, "f64", keep_pseudo=False)
    idx = torch.from_numpy(toks).cuda()
    out = f64(res.out.index_select(0, idx))
    st = f64(res.state)
    errs = {"out": rel_l2(out, ref["out"]), "state": rel_l2(st, ref["state"])}
    worst = {"out_worst_row": _rows_worst(out, ref["out"]), "state_worst_row": _rows_worst(st, ref["state"])}
    say(f"  forward on the sampled sequences: rel-L2 {errs}, worst rows {worst}")

    # commit: each sampled sequence's path from its root to the branch's last token
    L = TRUNK + BR
    path_nodes, path_ptr, spath_nodes = [], [0], []
    for i, s in enumerate(SAMPLE):
        local = list(range(FORK + 1)) + list(range(TRUNK, L))
        path_nodes += [int(seq_start[s]) + x for x in local]
        spath_nodes += [int(sstart[i]) + x for x in local]
        path_ptr.append(len(path_nodes))
    got = B.commit(k, log_gate, pd, sd, init, res.pseudo_v, np.array(path_ptr, np.int32),
                   np.array(path_nodes, np.int32), np.array(SAMPLE, np.int32), check=True)
    torch.cuda.synchronize()
    refc = oracle.commit(wl, "f64", path_ptr=np.array(path_ptr, np.int32), path_nodes=np.array(spath_nodes, np.int32),
                         path_seq=np.arange(len(SAMPLE), dtype=np.int32))
    errs["commit"] = rel_l2(f64(got), refc)
    worst["commit_worst_row"] = _rows_worst(f64(got), refc)
    say(f"  commit: rel-L2 {errs['commit']:.3e}")
    del res, got

    # ForkAttention: 32 query heads over 2 key/value heads
    ka, va = k[:, :2].contiguous(), v[:, :2].contiguous()
    att, _ = B.attention(q, ka, va, pd, sd, max_levels=cap["max_levels"], scale=D ** -0.5, check=True)
    torch.cuda.synchronize()
    aref = fork_attention(hq, hk[:, :2], hv[:, :2], spar, sstart, D ** -0.5)
    aout = f64(att.index_select(0, idx))
    errs["attention"] = rel_l2(aout, aref)
    worst["attention_worst_row"] = _rows_worst(aout, aref)
    say(f"  attention: rel-L2 {errs['attention']:.3e}")
    record_margin("large/524800x32x128", tol=TOL, row_tol=ROW_TOL, **errs, **worst)
    for kk, e in errs.items():
        assert e <= TOL, (kk, e)
    for kk, e in worst.items():
        assert e <= ROW_TOL, (kk, e)
