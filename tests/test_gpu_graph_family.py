"""Flat graphs over stream lengths (Flide, "Accelerating Decision Inference with
Exact State Forking", section 3.3.2) against the oracle.

A family of two buckets serves four rounds: two differently shaped rounds in
the small bucket (one captured graph, replayed for the second), a round that no
bucket holds (split along request boundaries into several replays) and a round
with one request larger than every bucket (run without a graph). Every
request's readout rows and states are compared with the fp64 oracle run on that
request alone, and bit for bit with an eager forward of the request alone
(results depend only on a request's own tokens). Eager forwards and host
synchronisations run between the replays.
"""
import numpy as np
import pytest
import torch

import oracle
from tree_forked_gated_amd import workloads as W

from gpu_helpers import record_margin, rel_l2, say

pytestmark = pytest.mark.gpu

H, D = 4, 128


def _decision(rng, L, n_q, qlen=(5, 70), nested=True):
    """A trunk of L tokens with n_q question branches forking from uniformly
    chosen trunk tokens (mostly mid-chunk), one of them nested in another
    question when asked for. Readouts: each question's last token; states: the
    leaves and the first question's fork token."""
    par = list(range(-1, L - 1))
    lasts, forks = [], []
    for b in range(n_q):
        bl = int(rng.integers(qlen[0], qlen[1] + 1))
        if nested and b == n_q - 1 and lasts:
            ft = int(rng.integers(L, len(par)))  # inside an earlier question
        else:
            ft = int(rng.integers(0, L))
        b0 = len(par)
        par += [ft] + list(range(b0, b0 + bl - 1))
        lasts.append(len(par) - 1)
        forks.append(ft)
    par = np.array(par, np.int32)
    leaves = W.leaves_of(par)
    states = np.unique(np.concatenate([leaves, [forks[0]]])).astype(np.int32)
    return par, np.array(lasts, np.int32), states


def _draft(rng):
    par = W.random_draft_tree(rng, int(rng.integers(8, 65)))
    leaves = W.leaves_of(par)
    return par, leaves[:8].astype(np.int32), leaves[:2].astype(np.int32)


def _request(seed, kind, **kw):
    from tree_forked_gated_amd.graphs import Request
    rng = np.random.default_rng(seed)
    par, outs, states = _decision(rng, **kw) if kind == "decision" else _draft(rng)
    n = par.shape[0]
    q, k, v, beta, g = W._values(rng, n, H, D, D, "bf16")
    init = W._init(rng, 1, H, D, D, True)
    f = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda().to(torch.bfloat16)
    req = Request(f(q), f(k), f(v), f(g), f(beta), par, torch.from_numpy(init[0]).cuda(), outs, states)
    wl = W.Workload(f"req{seed}", "bf16", par, np.array([0, n], np.int32), q, k, v, beta, g, init, outs, states)
    return req, wl


def _eager(req):
    from tree_forked_gated_amd import binding as B
    from tree_forked_gated_amd.graphs import request_needs
    nd = request_needs(req)
    return B.forward(req.q, req.k, req.v, req.log_gate, req.beta, req.parent, np.array([0, req.n], np.int32),
                     req.init_state.unsqueeze(0).contiguous(), out_rows=req.out_rows, state_rows=req.state_rows,
                     max_forks=nd.forks, max_levels=nd.levels, check=True)


def _bits(t):
    return t.contiguous().view(torch.int16 if t.dtype == torch.bfloat16 else torch.int32)


def _check_round(fam, name, reqs_wls, expect):
    reqs = [r for r, _ in reqs_wls]
    sched = fam.schedule(reqs)
    say(f"round {name}: tokens {[r.n for r in reqs]} -> schedule {sched}")
    assert [i for _, g in sched for i in g] == list(range(len(reqs)))  # each request once, in order
    assert expect(sched), sched
    res = fam.run(reqs)
    for (req, wl), got in zip(reqs_wls, res):
        eager = _eager(req)  # eager work between replays, and the bitwise twin
        torch.cuda.synchronize()
        assert torch.equal(_bits(got.out), _bits(eager.out)), (name, wl.name, "out")
        assert torch.equal(_bits(got.state), _bits(eager.state)), (name, wl.name, "state")
        ref = oracle.forward(wl, "f64", state_rows=wl.state_rows)
        e_out = rel_l2(got.out.float().cpu().numpy(), ref["out"][wl.out_rows])
        e_st = rel_l2(got.state.cpu().numpy(), ref["state"])
        record_margin(f"graph_family/{name}/{wl.name}", tol=1e-2, out=e_out, state=e_st, bucket=got.bucket)
        say(f"  {wl.name} (T={req.n}, bucket {got.bucket}, replay {got.replay}): out {e_out:.2e} state {e_st:.2e}")
        assert e_out <= 1e-2 and e_st <= 1e-2, (name, wl.name, e_out, e_st)
    return res


def test_graph_family_rounds_against_oracle():
    from tree_forked_gated_amd.graphs import Bucket, GraphFamily
    fam = GraphFamily([Bucket(T=1024, n_seq=6, max_forks=16, max_levels=3, n_out=40, n_state=40),
                       Bucket(T=3072, n_seq=8, max_forks=32, max_levels=4, n_out=96, n_state=96)],
                      H, D, D, torch.bfloat16)
    r1 = [_request(11, "decision", L=300, n_q=4), _request(12, "draft"), _request(13, "decision", L=150, n_q=3)]
    r2 = [_request(21, "draft"), _request(22, "decision", L=420, n_q=5), _request(23, "draft"),
          _request(24, "decision", L=130, n_q=2, nested=False)]
    r3 = [_request(31, "decision", L=1400, n_q=6), _request(32, "decision", L=1500, n_q=5),
          _request(33, "decision", L=900, n_q=4), _request(34, "draft")]
    r4 = [_request(41, "draft"), _request(42, "decision", L=3300, n_q=4), _request(43, "decision", L=200, n_q=3)]
    _check_round(fam, "small_a", r1, lambda sc: sc == [(0, [0, 1, 2])])
    assert fam.graphs[0] is not None and fam.replays[0] == 1
    _check_round(fam, "small_b", r2, lambda sc: sc == [(0, [0, 1, 2, 3])])
    assert fam.replays[0] == 2  # the second shape replayed the same captured graph
    # more tokens than the large bucket: several replays, split between requests
    _check_round(fam, "split", r3, lambda sc: len(sc) >= 2 and all(b is not None for b, _ in sc))
    # the 3300-token trunk exceeds every bucket: it alone runs without a graph
    _check_round(fam, "oversize", r4, lambda sc: [g for b, g in sc if b is None] == [[1]])
    assert sum(fam.replays) >= 5
