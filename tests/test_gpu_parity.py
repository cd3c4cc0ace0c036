"""HIP path vs the fp64 oracle, element by element, on seeded workloads.

Tolerances (relative L2 over each returned tensor): 1e-4 for fp32 inputs,
1e-2 for bf16 inputs (the spec bar). Sizes span several 64-token chunks,
ragged chunk tails, forks in the middle of chunks, nested forks, tree chunks
of every size up to 64 and several heads.
"""
import numpy as np
import pytest

from tree_forked_gated_amd import workloads as W

from gpu_helpers import f64, oracle_ref, record_margin, rel_l2, run_forward, say, to_device, tol

pytestmark = pytest.mark.gpu


def _check(wl, name, dv_tile=0, pseudo=True):
    leaves = W.leaves_of(wl.parent)
    rows = wl.state_rows if wl.state_rows.size else leaves
    say(f"parity {name}: T={wl.T} H={wl.H} Dk={wl.Dk} Dv={wl.Dv} dtype={wl.dtype} dv_tile={dv_tile}")
    res, _ = run_forward(wl, keep_pseudo=pseudo, state_rows=rows, dv_tile=dv_tile)
    ref = oracle_ref(wl, state_rows=rows)
    ref_out = ref["out"] if wl.out_rows is None else ref["out"][wl.out_rows]
    errs = {"out": rel_l2(f64(res.out), ref_out), "state": rel_l2(f64(res.state), ref["state"])}
    if pseudo:
        errs["pseudo_v"] = rel_l2(f64(res.pseudo_v), ref["pseudo_v"])
    say(f"  rel-L2 {errs}")
    record_margin(f"parity/{name}", tol=tol(wl), **errs)
    for k, e in errs.items():
        assert e <= tol(wl), (name, k, e)
    return res, ref


def test_tiny_tree_fp32():
    wl = W.tiny_tree()
    res, ref = _check(wl, "tiny_tree")
    # the five leaf states of the workload
    assert res.state.shape[0] == 5


@pytest.mark.parametrize("seed,Dk,Dv", [(1, 16, 16), (2, 32, 48), (3, 64, 32), (4, 64, 64), (5, 16, 128)])
def test_random_fp32(seed, Dk, Dv):
    wl = W.random_small(seed, n_seq=4, H=2, Dk=Dk, Dv=Dv, dtype="f32", max_len=300)
    _check(wl, f"random_f32[{seed}]")


@pytest.mark.parametrize("seed,Dk,Dv", [(6, 32, 32), (7, 64, 64), (8, 128, 128), (9, 128, 64), (10, 128, 16)])
def test_random_bf16(seed, Dk, Dv):
    wl = W.random_small(seed, n_seq=4, H=2, Dk=Dk, Dv=Dv, dtype="bf16", max_len=300)
    _check(wl, f"random_bf16[{seed}]")


@pytest.mark.parametrize("dtype,Dk,Dv,seed", [("f32", 64, 48, 21), ("bf16", 128, 128, 22), ("bf16", 64, 32, 23)])
def test_degenerate_gates_and_betas(dtype, Dk, Dv, seed):
    """The extremes the recurrence admits, mixed into a random stream: log
    gates of 0 (no decay) and of -40 (the state all but cleared: alpha =
    4e-18), and beta of 0 (the token writes nothing) and of 1 (a full
    replacement along its key). Forward outputs, leaf states and pseudo-values,
    and the commit of every sequence's deepest path, against the oracle."""
    import oracle
    import torch
    from tree_forked_gated_amd import binding as B
    wl = W.random_small(seed, n_seq=4, H=2, Dk=Dk, Dv=Dv, dtype=dtype, max_len=300)
    rng = np.random.default_rng(seed)
    pick = rng.random(wl.log_gate.shape)
    wl.log_gate = np.where(pick < 0.15, 0.0, np.where(pick < 0.25, -40.0, wl.log_gate)).astype(np.float32)
    pick = rng.random(wl.beta.shape)
    wl.beta = np.where(pick < 0.15, 0.0, np.where(pick < 0.3, 1.0, wl.beta)).astype(np.float32)
    res, ref = _check(wl, f"degenerate_{dtype}[{seed}]")
    ptr, nodes = [0], []
    for s_ in range(wl.n_seq):
        a, b = int(wl.seq_start[s_]), int(wl.seq_start[s_ + 1])
        deepest = max((W.root_path(wl.parent, t) for t in range(a, b)), key=len, default=[])
        nodes += deepest
        ptr.append(len(nodes))
    ptr, nodes, seqs = np.array(ptr, np.int32), np.array(nodes, np.int32), np.arange(wl.n_seq, dtype=np.int32)
    d = to_device(wl)
    got = B.commit(d["k"], d["log_gate"], d["parent_idx"], d["seq_start"], d["init_state"], res.pseudo_v, ptr, nodes,
                   seqs, check=True)
    torch.cuda.synchronize()
    e = rel_l2(f64(got), oracle.commit(wl, "f64", path_ptr=ptr, path_nodes=nodes, path_seq=seqs))
    say(f"  commit rel-L2 {e:.3e}")
    assert e <= tol(wl), e


def test_chains_bf16():
    wl = W.chains(n_seq=3, L=333, H=3, D=128)
    _check(wl, "chains")


def test_decision_round_bf16():
    wl = W.decision_round(n_req=2, trunk=300, n_branch=5, blen=32, H=2, D=128)
    _check(wl, "decision")


def test_draft_trees_bf16():
    wl = W.draft_trees(n_seq=8, n_nodes=64, H=2, D=128)
    _check(wl, "draft")


def test_mixed_forest_bf16():
    wl = W.mixed_forest(total=4000, H=2, D=128, trunk_range=(100, 900), branch_count=(1, 12), branch_len=(1, 90))
    _check(wl, "mixed")


def test_short_sequences_with_rows_bf16():
    """Every sequence fits one chunk (the planner's one-pass path): readout rows
    in shuffled order, state rows at leaves and inner nodes, an empty sequence
    and one-token sequences among draft trees of up to 64 tokens."""
    rng = np.random.default_rng(41)
    sizes = [64, 1, 0, 37, 64, 2, 17, 50, 1]
    parents, starts, used = [], [0], 0
    for n in sizes:
        lp = W.random_draft_tree(rng, n) if n else np.zeros(0, np.int32)
        parents.append(np.where(lp < 0, -1, lp + used).astype(np.int32))
        used += n
        starts.append(used)
    parent = np.concatenate(parents).astype(np.int32)
    seq_start = np.array(starts, np.int32)
    T, H, D = used, 2, 128
    q, k, v, beta, g = W._values(rng, T, H, D, D, "bf16")
    init = W._init(rng, len(sizes), H, D, D, True)
    out_rows = rng.permutation(T)[: T // 2].astype(np.int32)
    inner = np.setdiff1d(np.unique(parent[parent >= 0]), W.leaves_of(parent))[:9]
    state_rows = rng.permutation(np.concatenate([W.leaves_of(parent), inner])).astype(np.int32)
    wl = W.Workload("short_rows", "bf16", parent, seq_start, q, k, v, beta, g, init, out_rows, state_rows)
    _check(wl, "short_rows")


@pytest.mark.parametrize("n_nodes", [1, 2, 17, 63, 64])
def test_tree_chunk_sizes_fp32(n_nodes):
    wl = W.draft_trees(n_seq=3, n_nodes=n_nodes, H=1, D=16)
    wl.dtype = "f32"
    _check(wl, f"tree{n_nodes}")


@pytest.mark.parametrize("dv_tile", [16, 32, 64])
def test_dv_tiles_bitwise_identical(dv_tile):
    wl = W.random_small(21, n_seq=4, H=2, Dk=128, Dv=128, dtype="bf16", max_len=200)
    base, _ = run_forward(wl, keep_pseudo=True, state_rows=W.leaves_of(wl.parent), dv_tile=16)
    say(f"dv tile {dv_tile} vs 16")
    res, _ = run_forward(wl, keep_pseudo=True, state_rows=W.leaves_of(wl.parent), dv_tile=dv_tile)
    assert np.array_equal(res.out.view(dtype=base.out.dtype).cpu().float().numpy(), base.out.cpu().float().numpy())
    assert np.array_equal(res.state.cpu().numpy(), base.state.cpu().numpy())
    assert np.array_equal(res.pseudo_v.cpu().numpy(), base.pseudo_v.cpu().numpy())


def test_planned_walk_is_bitwise_the_full_forward():
    """GDN_FWD_PLANNED reuses the workspace's metadata: the walk alone gives the
    same bits as a forward that plans first; a workspace planned for other
    sizes is refused on the device (GDN_DEV_NOT_PLANNED) instead of walked."""
    import torch
    from tree_forked_gated_amd import binding as B
    wl = W.random_small(31, n_seq=4, H=2, Dk=64, Dv=64, dtype="bf16", max_len=300)
    rows = W.leaves_of(wl.parent)
    say("planned walk vs full forward")
    base, d = run_forward(wl, keep_pseudo=True, state_rows=rows)
    ws = base.workspace
    out2 = torch.empty_like(base.out)
    st2 = torch.empty_like(base.state)
    pv2 = torch.empty_like(base.pseudo_v)
    cap = B.capacities(wl.parent, wl.seq_start)
    B.forward(d["q"], d["k"], d["v"], d["log_gate"], d["beta"], d["parent_idx"], d["seq_start"], d["init_state"],
              state_rows=rows, keep_pseudo=True, workspace=ws, out=out2, state_out=st2, pseudo_v=pv2,
              max_forks=cap["max_forks"], max_levels=cap["max_levels"], planned=True, check=True)
    torch.cuda.synchronize()
    assert torch.equal(out2, base.out) and torch.equal(st2, base.state) and torch.equal(pv2, base.pseudo_v)
    # fewer state rows than the plan was built for: refused, nothing written
    st3 = torch.full_like(base.state[:1], 7.0)
    B.forward(d["q"], d["k"], d["v"], d["log_gate"], d["beta"], d["parent_idx"], d["seq_start"], d["init_state"],
              state_rows=rows[:1], keep_pseudo=False, workspace=ws, state_out=st3,
              max_forks=cap["max_forks"], max_levels=cap["max_levels"], planned=True)
    code, _ = B.check_error(ws)
    assert code == 8
    assert bool((st3 == 7.0).all())


@pytest.mark.parametrize("seed", [100, 107, 113, 121, 128, 136])
def test_random_forests_dk128_every_tile(seed):
    """Random chains, draft trees and nested forests at d_k = 128 in bf16 (the
    pipelined walk), every d_v tile width that divides d_v, all leaf states."""
    rng = np.random.default_rng(seed)
    Dv = int(rng.choice([16, 32, 64, 128]))
    H = int(rng.integers(1, 4))
    wl = W.random_small(seed, n_seq=int(rng.integers(1, 6)), H=H, Dk=128, Dv=Dv, dtype="bf16", max_len=400)
    for dv_tile in [0] + [t for t in (16, 32, 64) if Dv % t == 0]:
        _check(wl, f"random_dk128[{seed}] tile {dv_tile}", dv_tile=dv_tile)
