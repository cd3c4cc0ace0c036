"""Flat-graph replay: one captured forward per size bucket serves every tree
that fits the bucket (Flide, "Accelerating Decision Inference with Exact State
Forking", §3.3). The replayed kernels rebuild the tree metadata on the device,
so a replay for a new tree gives the same bits as an eager forward of that tree
with the same capacities. Replays alternate with eager work and host
synchronisation, and every replay is checked against its eager twin."""
import numpy as np
import pytest
import torch

from tree_forked_gated_amd import workloads as W

from gpu_helpers import say

pytestmark = pytest.mark.gpu


def _random_parents(rng, L, p_fork):
    """Parents of one sequence: mostly the previous token, sometimes a random
    earlier token or the initial state (a new branch)."""
    par = np.empty(L, dtype=np.int32)
    par[0] = -1
    for i in range(1, L):
        par[i] = i - 1 if rng.random() > p_fork else int(rng.integers(-1, i))
    return par


def _round(seed, lens, H, D, dtype, n_out, n_state):
    rng = np.random.default_rng(seed)
    parents, starts, used = [], [0], 0
    for L in lens:
        lp = _random_parents(rng, L, 0.08 if L > 64 else 0.5)
        parents.append(np.where(lp < 0, -1, lp + used).astype(np.int32))
        used += L
        starts.append(used)
    T = used
    q, k, v, beta, g = W._values(rng, T, H, D, D, dtype)
    return {"parent": np.concatenate(parents), "seq_start": np.array(starts, dtype=np.int32), "q": q, "k": k,
            "v": v, "beta": beta, "g": g, "init": W._init(rng, len(lens), H, D, D, True),
            "out_rows": np.sort(rng.choice(T, n_out, replace=False)).astype(np.int32),
            "state_rows": rng.choice(T, n_state, replace=False).astype(np.int32)}


def _dev(r, tdt):
    f = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda().to(tdt).contiguous()
    i = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()
    return {"q": f(r["q"]), "k": f(r["k"]), "v": f(r["v"]), "log_gate": f(r["g"]), "beta": f(r["beta"]),
            "parent_idx": i(r["parent"]), "seq_start": i(r["seq_start"]),
            "init_state": torch.from_numpy(np.ascontiguousarray(r["init"], dtype=np.float32)).cuda(),
            "out_rows": i(r["out_rows"]), "state_rows": i(r["state_rows"])}


def _bits(t):
    return t.contiguous().view(torch.int16 if t.dtype == torch.bfloat16 else torch.int32)


def _same(a, b):
    return bool(torch.equal(_bits(a), _bits(b)))


@pytest.mark.parametrize("dtype,D,H", [("bf16", 128, 4), ("f32", 32, 2)])
def test_graph_replay_serves_every_tree_in_the_bucket(dtype, D, H):
    from tree_forked_gated_amd import binding as B
    lens = [300, 64, 150]
    n_out, n_state = 48, 12
    rounds = [_round(s, lens, H, D, dtype, n_out, n_state) for s in (11, 12, 13)]
    caps = [B.capacities(r["parent"], r["seq_start"]) for r in rounds]
    mf = max(c["max_forks"] for c in caps)
    ml = max(c["max_levels"] for c in caps)
    say(f"graph replay {dtype} D={D} H={H}: T={sum(lens)} capacities forks {mf} levels {ml} "
        f"(per round {[(c['max_forks'], c['max_levels']) for c in caps]})")
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    fg = B.ForwardGraph(sum(lens), H, D, D, len(lens), tdt, max_forks=mf, max_levels=ml, n_out=n_out,
                        n_state=n_state, keep_pseudo=True)
    d0 = _dev(rounds[0], tdt)
    fg.load(**d0)
    fg.capture()
    for step, i in enumerate([1, 0, 2, 1, 2]):
        d = _dev(rounds[i], tdt)
        fg.load(**d)
        fg.replay()
        # eager work between replays: the reference forward of the same round
        ref = B.forward(d["q"], d["k"], d["v"], d["log_gate"], d["beta"], d["parent_idx"], d["seq_start"],
                        d["init_state"], out_rows=d["out_rows"], state_rows=d["state_rows"], keep_pseudo=True,
                        max_forks=mf, max_levels=ml)
        torch.cuda.synchronize()
        fg.check()
        B.raise_device_error(ref.workspace)
        say(f"  replay {step}: round {i}")
        assert _same(fg.out, ref.out), f"replay {step} (round {i}): outputs differ"
        assert _same(fg.state_out, ref.state), f"replay {step} (round {i}): states differ"
        assert _same(fg.pseudo_v, ref.pseudo_v), f"replay {step} (round {i}): pseudo-values differ"


def test_graph_replay_draft_trees_with_commit():
    from tree_forked_gated_amd import binding as B
    n_seq, n_nodes, H, D = 8, 64, 4, 128
    rounds = [W.draft_trees(seed=s, n_seq=n_seq, n_nodes=n_nodes, H=H, D=D) for s in (21, 22, 23)]
    T = n_seq * n_nodes
    say(f"graph replay draft trees {n_seq}x{n_nodes} H={H}: path lengths "
        f"{[int(r.path_ptr[-1]) for r in rounds]}")
    fg = B.ForwardGraph(T, H, D, D, n_seq, torch.bfloat16, max_forks=0, max_levels=1, keep_pseudo=True,
                        n_path=n_seq, path_capacity=T)

    def dev(wl):
        f = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda().to(torch.bfloat16)
        i = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()
        return {"q": f(wl.q), "k": f(wl.k), "v": f(wl.v), "log_gate": f(wl.log_gate), "beta": f(wl.beta),
                "parent_idx": i(wl.parent), "seq_start": i(wl.seq_start),
                "init_state": torch.from_numpy(np.ascontiguousarray(wl.init_state, dtype=np.float32)).cuda(),
                "path_ptr": i(wl.path_ptr), "path_nodes": i(wl.path_nodes), "path_seq": i(wl.path_seq)}

    fg.load(**dev(rounds[0]))
    fg.capture()
    for step, i in enumerate([2, 1, 0, 2]):
        d = dev(rounds[i])
        fg.load(**d)
        fg.replay()
        ref = B.forward(d["q"], d["k"], d["v"], d["log_gate"], d["beta"], d["parent_idx"], d["seq_start"],
                        d["init_state"], keep_pseudo=True, max_forks=0, max_levels=1)
        st = B.commit(d["k"], d["log_gate"], d["parent_idx"], d["seq_start"], d["init_state"], ref.pseudo_v,
                      d["path_ptr"], d["path_nodes"], d["path_seq"])
        torch.cuda.synchronize()
        fg.check()
        B.raise_device_error(ref.workspace)
        say(f"  replay {step}: round {i}")
        assert _same(fg.out, ref.out), f"replay {step} (round {i}): outputs differ"
        assert _same(fg.pseudo_v, ref.pseudo_v), f"replay {step} (round {i}): pseudo-values differ"
        assert _same(fg.committed, st), f"replay {step} (round {i}): committed states differ"


def test_graph_replay_reports_a_tree_beyond_its_bucket():
    """A round that needs more levels than the bucket holds is reported through
    the device error word (the walk then computes nothing); the next round that
    fits replays correctly from the same graph."""
    from tree_forked_gated_amd import binding as B
    lens, H, D = [300, 64, 150], 4, 128
    rounds = {s: _round(s, lens, H, D, "bf16", 48, 12) for s in (11, 12)}
    caps = {s: B.capacities(r["parent"], r["seq_start"]) for s, r in rounds.items()}
    mf = max(c["max_forks"] for c in caps.values())
    ml = caps[11]["max_levels"]
    assert caps[12]["max_levels"] > ml, caps
    say(f"bucket: forks {mf}, levels {ml}; the round of seed 12 needs {caps[12]['max_levels']} levels")
    fg = B.ForwardGraph(sum(lens), H, D, D, len(lens), torch.bfloat16, max_forks=mf, max_levels=ml, n_out=48,
                        n_state=12, keep_pseudo=True)
    fg.load(**_dev(rounds[11], torch.bfloat16))
    fg.capture()
    fg.load(**_dev(rounds[12], torch.bfloat16))
    fg.replay()
    torch.cuda.synchronize()
    with pytest.raises(B.GdnDeviceError) as ei:
        fg.check()
    assert ei.value.code == 5, ei.value  # level capacity
    d = _dev(rounds[11], torch.bfloat16)
    fg.load(**d)
    fg.replay()
    ref = B.forward(d["q"], d["k"], d["v"], d["log_gate"], d["beta"], d["parent_idx"], d["seq_start"],
                    d["init_state"], out_rows=d["out_rows"], state_rows=d["state_rows"], keep_pseudo=True,
                    max_forks=mf, max_levels=ml)
    torch.cuda.synchronize()
    fg.check()
    assert _same(fg.out, ref.out) and _same(fg.state_out, ref.state) and _same(fg.pseudo_v, ref.pseudo_v)
