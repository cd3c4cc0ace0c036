"""Exactness properties of the HIP path that hold bit for bit.

Batch composition: a sequence's outputs and states do not depend on which
other sequences share the stream, or where in the stream it sits (Flide's
state forking: a question's result is the same inside the round as alone).

Branch alone: a branch walked inside the stream from its fork state gives the
same bits as the branch run as a sequence of its own whose initial state is
that fork state (read back through a state row at the fork token). Branches
here are longer than one chunk so that both runs cut them into the same
64-token chunks from the branch's first token.

Repeated calls: the forward, ForkAttention and the commit, run again on the
same inputs into outputs prefilled with NaN or 7, give the same bits.
"""
import numpy as np
import pytest
import torch

from tree_forked_gated_amd import workloads as W

from gpu_helpers import run_forward, say

pytestmark = pytest.mark.gpu


def _seq_values(seed, n, H, D, dtype):
    rng = np.random.default_rng(seed)
    q, k, v, beta, g = W._values(rng, n, H, D, D, dtype)
    init = W._init(rng, 1, H, D, D, True)[0]
    return q, k, v, beta, g, init


def _forest(seed, trunk, branches):
    """Local parents of a trunk (chain) plus branches given as (fork token, length)."""
    par = list(range(-1, trunk - 1))
    for ft, bl in branches:
        b0 = len(par)
        par += [ft] + list(range(b0, b0 + bl - 1))
    return np.array(par, dtype=np.int32)


def _draft(seed, n):
    rng = np.random.default_rng(seed)
    par = [-1]
    for i in range(1, n):
        par.append(int(rng.integers(-1, i)))
    return np.array(par, dtype=np.int32)


def _stream(seqs, H, D, dtype):
    """Concatenate sequences given as (local parents, seed); returns the workload
    and the global offset of each sequence."""
    parents, offs, used = [], [], 0
    cols = {k: [] for k in ("q", "k", "v", "beta", "g")}
    inits = []
    for lp, seed in seqs:
        n = lp.shape[0]
        q, k, v, beta, g, init = _seq_values(seed, n, H, D, dtype)
        for name, arr in zip(("q", "k", "v", "beta", "g"), (q, k, v, beta, g)):
            cols[name].append(arr)
        inits.append(init)
        parents.append(np.where(lp < 0, -1, lp + used).astype(np.int32))
        offs.append(used)
        used += n
    seq_start = np.array(offs + [used], dtype=np.int32)
    parent = np.concatenate(parents)
    wl = W.Workload(f"stream_{used}", dtype, parent, seq_start, np.concatenate(cols["q"]), np.concatenate(cols["k"]),
                    np.concatenate(cols["v"]), np.concatenate(cols["beta"]), np.concatenate(cols["g"]),
                    np.stack(inits), None, W.leaves_of(parent))
    return wl, offs


def _bits(t):
    return t.detach().cpu().contiguous().view(torch.int16 if t.dtype == torch.bfloat16 else torch.int32).numpy()


@pytest.mark.parametrize("dtype,D", [("bf16", 128), ("f32", 32)])
def test_batch_composition_bitwise(dtype, D):
    H = 2
    A = (_forest(1, 300, [(299, 40), (150, 70), (17, 5)]), 11)
    B = (_forest(2, 200, [(63, 64), (64, 65), (199, 9), (100, 130)]), 22)
    C = (_draft(3, 64), 33)
    E = (_forest(4, 90, [(89, 12)]), 44)
    x, ox = _stream([A, B, C], H, D, dtype)
    y, oy = _stream([E, C, B, A], H, D, dtype)
    nb = B[0].shape[0]
    say(f"batch composition {dtype} D={D}: B at {ox[1]} and {oy[2]}, T={x.T} and {y.T}")
    rx, _ = run_forward(x, keep_pseudo=True)
    ry, _ = run_forward(y, keep_pseudo=True)
    sx, sy = slice(ox[1], ox[1] + nb), slice(oy[2], oy[2] + nb)
    assert np.array_equal(_bits(rx.out[sx]), _bits(ry.out[sy]))
    assert np.array_equal(_bits(rx.pseudo_v[sx]), _bits(ry.pseudo_v[sy]))
    # leaf states of B: the state rows are the leaves in stream order
    lx = np.nonzero((x.state_rows >= ox[1]) & (x.state_rows < ox[1] + nb))[0]
    ly = np.nonzero((y.state_rows >= oy[2]) & (y.state_rows < oy[2] + nb))[0]
    assert lx.size == ly.size > 0
    assert np.array_equal(_bits(rx.state[lx]), _bits(ry.state[ly]))


@pytest.mark.parametrize("dtype,D", [("bf16", 128), ("f32", 32)])
def test_branch_in_stream_equals_branch_alone(dtype, D):
    H = 2
    trunk = 300
    branches = [(150, 130), (299, 70), (63, 66)]  # no branch directly follows its fork token
    lp = _forest(5, trunk, branches)
    x, _ = _stream([(lp, 55)], H, D, dtype)
    forks = np.array([b[0] for b in branches], dtype=np.int32)
    say(f"branch alone {dtype} D={D}: T={x.T}, forks {forks.tolist()}")
    rx, _ = run_forward(x, keep_pseudo=True, state_rows=forks)
    start = trunk
    for i, (ft, bl) in enumerate(branches):
        sl = slice(start, start + bl)
        alone = W.Workload(f"branch_{i}", dtype, np.array([-1] + list(range(bl - 1)), np.int32),
                           np.array([0, bl], np.int32), x.q[sl], x.k[sl], x.v[sl], x.beta[sl], x.log_gate[sl],
                           rx.state[i:i + 1].cpu().numpy(), None, np.array([bl - 1], np.int32))
        ra, _ = run_forward(alone, keep_pseudo=True)
        assert np.array_equal(_bits(rx.out[sl]), _bits(ra.out)), i
        assert np.array_equal(_bits(rx.pseudo_v[sl]), _bits(ra.pseudo_v)), i
        start += bl


def test_repeated_calls_are_bitwise_equal():
    """Races or reads of unwritten memory would show as differences between
    repeated calls on the same inputs. The forward over a nested-forest stream
    (several fork levels, items claimed dynamically), planned and not,
    ForkAttention over the same stream, and the commit of draft-tree paths each
    run again into outputs prefilled with NaN and with 7, and agree with the
    first call bit for bit."""
    from gpu_helpers import to_device
    from tree_forked_gated_amd import binding as B
    wl = W.mixed_forest(seed=91, total=12000, H=8, D=128)
    d = to_device(wl)
    rows = W.leaves_of(wl.parent)
    cap = B.capacities(wl.parent, wl.seq_start)
    args = (d["q"], d["k"], d["v"], d["log_gate"], d["beta"], d["parent_idx"], d["seq_start"], d["init_state"])
    kw = dict(state_rows=rows, keep_pseudo=True, max_forks=cap["max_forks"], max_levels=cap["max_levels"])
    first = B.forward(*args, check=True, **kw)
    kq, vq = d["k"][:, :2].contiguous(), d["v"][:, :2].contiguous()
    att0, aws = B.attention(d["q"], kq, vq, d["parent_idx"], d["seq_start"], max_levels=cap["max_levels"], check=True)
    dt = W.draft_trees(seed=92, n_seq=16, n_nodes=64, H=8, D=128)
    dd = to_device(dt)
    cres = B.forward(dd["q"], dd["k"], dd["v"], dd["log_gate"], dd["beta"], dd["parent_idx"], dd["seq_start"],
                     dd["init_state"], state_rows=np.zeros(0, np.int32), keep_pseudo=True, check=True,
                     **B.capacities(dt.parent, dt.seq_start))
    cargs = (dd["k"], dd["log_gate"], dd["parent_idx"], dd["seq_start"], dd["init_state"], cres.pseudo_v,
             dt.path_ptr, dt.path_nodes, dt.path_seq)
    com0 = B.commit(*cargs, check=True)
    torch.cuda.synchronize()
    say(f"repeat runs: forest T={wl.T} ({cap['max_levels']} levels), draft trees {dt.n_path} paths")
    for fill, planned in ((float("nan"), False), (7.0, True), (float("nan"), True)):
        out, st, pv = (torch.full_like(x, fill) for x in (first.out, first.state, first.pseudo_v))
        B.forward(*args, out=out, state_out=st, pseudo_v=pv, workspace=first.workspace, planned=planned, check=True,
                  **kw)
        att = torch.full_like(att0, fill)
        B.attention(d["q"], kq, vq, d["parent_idx"], d["seq_start"], max_levels=cap["max_levels"], workspace=aws,
                    out=att, planned=planned, check=True)
        com = torch.full_like(com0, fill)
        B.commit(*cargs, out_state=com, check=True)
        torch.cuda.synchronize()
        assert torch.equal(out, first.out) and torch.equal(st, first.state) and torch.equal(pv, first.pseudo_v), \
            (fill, planned, "forward")
        assert torch.equal(att, att0), (fill, planned, "attention")
        assert torch.equal(com, com0), (fill, planned, "commit")
