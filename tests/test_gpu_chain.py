"""Fused chain verify + commit with the deferred state write (gdn_chain_step)
against the speculative chain-round oracle (oracle/chain.py).

Eight rounds of chain drafts per sequence, with seeded accepted counts
(including rounds that accept nothing and rounds that accept the whole draft),
with drafts of 4, 7, 12 and 32 tokens and d_v of 16 to 128 (also unlike d_k).
Every round's outputs and pseudo-values, and the committed state it starts from
(state_out), are compared with the oracle: with the state written every round
(history capacity 0), with a short history that flushes every few rounds, and
with a history long enough that nothing flushes until a forced flush. After
the forced flush the checkpoint itself must hold the committed state. Rounds
replayed from captured graphs equal eager rounds bit for bit. A bad accepted
count is reported on the device and its sequence skipped.
"""
import numpy as np
import pytest
import torch

from oracle.chain import chain_rounds
from tree_forked_gated_amd import workloads as W

from gpu_helpers import record_margin, rel_l2, say

pytestmark = pytest.mark.gpu


def _draft(rng, n_seq, N, H, D, dtype, Dv=None):
    q, k, v, beta, g = W._values(rng, n_seq * N, H, D, D if Dv is None else Dv, dtype)
    sh = lambda a: a.reshape((n_seq, N) + a.shape[1:])
    return {"q": sh(q), "k": sh(k), "v": sh(v), "beta": sh(beta), "log_gate": sh(g)}


@pytest.mark.parametrize("dtype,D,cap", [("bf16", 128, 0), ("bf16", 128, 6), ("bf16", 128, 64), ("f32", 32, 5),
                                         ("f32", 64, 0)])
def test_chain_rounds_against_oracle(dtype, D, cap):
    _rounds_against_oracle(dtype, D, cap, n_seq=5, N=4, H=3, R=8, seed=100 + cap + D, tag="")


@pytest.mark.parametrize("dtype,D,cap", [("bf16", 128, 0), ("bf16", 128, 30), ("f32", 64, 13)])
def test_chain_rounds_long_drafts(dtype, D, cap):
    """Drafts of 12 tokens (three times the benched length), with histories
    that flush every few rounds (30, 13) or never hold anything (0)."""
    _rounds_against_oracle(dtype, D, cap, n_seq=4, N=12, H=2, R=5, seed=200 + cap + D, tag="n12_")


@pytest.mark.parametrize("dtype,D,Dv,cap,N", [("bf16", 128, 80, 40, 32), ("f32", 32, 48, 0, 7), ("bf16", 64, 16, 9, 3)])
def test_chain_rounds_ragged_dv_and_longest_draft(dtype, D, Dv, cap, N):
    """d_v of 80, 48 and 16 (a last block of 16 rows of S), the longest draft
    (32 tokens) with a 40-token history (paths of up to 72 tokens, five tiles
    with a ragged last one), and a 7-token draft without history."""
    _rounds_against_oracle(dtype, D, cap, n_seq=3, N=N, H=2, R=5, seed=400 + cap + Dv, tag="dv_", Dv=Dv)


@pytest.mark.parametrize("cap", [0, 16])
def test_chain_rounds_full_size(cap):
    """The benched size: 64 sequences x 32 heads x d 128, 4-token drafts, bf16,
    with the state written every round (capacity 0) and with the 16-token
    deferred history; three rounds and the forced flush, every sequence and
    head against the oracle."""
    _rounds_against_oracle("bf16", 128, cap, n_seq=64, N=4, H=32, R=3, seed=300 + cap, tag="full_")


def _rounds_against_oracle(dtype, D, cap, n_seq, N, H, R, seed, tag, Dv=None):
    from tree_forked_gated_amd import binding as B
    rng = np.random.default_rng(seed)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    Dv = D if Dv is None else Dv
    S0 = W._init(rng, n_seq, H, Dv, D, True)
    rounds = [_draft(rng, n_seq, N, H, D, dtype, Dv) for _ in range(R)]
    acc = [rng.integers(0, N + 1, n_seq) for _ in range(R)]
    if R >= 4:  # a round that accepts nothing and one that accepts every draft
        acc[2][:] = 0
        acc[3][:] = N
    else:  # half the sequences accept nothing in one round, the other half everything in the next
        acc[R - 2][: n_seq // 2] = 0
        acc[R - 1][n_seq // 2:] = N
    # accepted[r] is what the sampler keeps of draft r; round r + 1 commits it
    ref, S_end = chain_rounds(S0, rounds, acc)
    cr = B.ChainRounds(torch.from_numpy(S0).cuda(), N, cap, tdt, keep_state=True)
    tol = 1e-2 if dtype == "bf16" else 1e-4
    say(f"chain rounds {dtype} Dk={D} Dv={Dv} hist_cap={cap}: {n_seq} sequences x {R} rounds of {N} draft tokens")
    f = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.float32)).cuda().to(tdt).contiguous()
    worst = {"out": 0.0, "pseudo_v": 0.0, "state": 0.0}
    for r in range(R + 1):
        prev_acc = np.zeros(n_seq, np.int32) if r == 0 else acc[r - 1].astype(np.int32)
        last = r == R
        draft = {kk: f(x) for kk, x in rounds[min(r, R - 1)].items()}
        out, pv = cr.step(draft, torch.from_numpy(prev_acc).cuda(), flush=last, check=True)
        torch.cuda.synchronize()
        want_state = S_end if last else ref[r]["start_state"]
        e = {"state": rel_l2(cr.state.cpu().numpy(), want_state)}
        if not last:
            e["out"] = rel_l2(out.float().cpu().numpy(), ref[r]["out"])
            e["pseudo_v"] = rel_l2(pv.cpu().numpy(), ref[r]["pseudo_v"])
        for kk, x in e.items():
            worst[kk] = max(worst[kk], x)
            assert x <= tol, (r, kk, x)
    # the forced flush leaves the committed state in the checkpoint and an empty history
    ck = rel_l2(cr.ckpt.cpu().numpy(), S_end)
    say(f"  worst rel-L2 over the rounds {worst}; checkpoint after the flush {ck:.2e}")
    record_margin(f"chain/{tag}{dtype}_d{D}_dv{Dv}_cap{cap}", tol=tol, checkpoint=ck, **worst)
    assert ck <= tol
    assert int(cr.hist_len[1 - cr.cur].abs().sum()) == 0


@pytest.mark.parametrize("cap", [0, 6])
def test_chain_rounds_replayed_from_graphs(cap):
    """TreeWY section 4: a chain round is one graph-capturable kernel, since the
    accepted counts and history lengths are device data. Two graphs are
    captured, one per parity of the alternating buffers, and replayed for eight
    rounds with new drafts and accepted counts copied into their static inputs
    (eager work and host synchronisation between replays); every round's
    outputs, pseudo-values and starting state equal an eager run's bit for bit
    and match the oracle. With capacity 6 the same two graphs append to the
    history in some rounds and flush it in others."""
    from tree_forked_gated_amd import binding as B
    rng = np.random.default_rng(500 + cap)
    n_seq, N, H, D, R = 8, 4, 4, 128, 8
    S0 = W._init(rng, n_seq, H, D, D, True)
    rounds = [_draft(rng, n_seq, N, H, D, "bf16") for _ in range(R)]
    acc = [rng.integers(0, N + 1, n_seq) for _ in range(R)]
    ref, _ = chain_rounds(S0, rounds, acc)
    f = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.float32)).cuda().to(torch.bfloat16).contiguous()
    init = torch.from_numpy(S0).cuda()
    cr_e = B.ChainRounds(init, N, cap, torch.bfloat16, keep_state=True)
    cr_g = B.ChainRounds(init, N, cap, torch.bfloat16, keep_state=True)
    stat = [{kk: f(x) for kk, x in rounds[0].items()} for _ in range(2)]  # static drafts, by parity
    eager = [{kk: f(x) for kk, x in rounds[0].items()} for _ in range(2)]
    a_g = torch.zeros(n_seq, dtype=torch.int32, device="cuda")
    cr_g.prev_k, cr_g.prev_g = stat[1]["k"], stat[1]["log_gate"]
    graphs = [torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph()]
    torch.cuda.synchronize()
    for par in range(2):
        with B.capture_guard(), torch.cuda.graph(graphs[par]):
            cr_g.step(stat[par], a_g)
    assert cr_g.cur == 0
    say(f"chain rounds from graphs, hist_cap={cap}: {n_seq} sequences x {R} rounds")
    for r in range(R):
        par = r % 2
        prev_acc = np.zeros(n_seq, np.int32) if r == 0 else acc[r - 1].astype(np.int32)
        for kk, x in rounds[r].items():
            stat[par][kk].copy_(f(x))
            eager[par][kk].copy_(f(x))
        a_g.copy_(torch.from_numpy(prev_acc))
        graphs[par].replay()
        torch.cuda.synchronize()
        out_g, pv_g, st_g = cr_g.out[par].clone(), cr_g.pv[par].clone(), cr_g.state.clone()
        out_e, pv_e = cr_e.step(eager[par], torch.from_numpy(prev_acc).cuda(), check=True)
        torch.cuda.synchronize()
        assert torch.equal(out_g, out_e) and torch.equal(pv_g, pv_e), f"round {r}: replay differs from eager"
        assert torch.equal(st_g, cr_e.state), f"round {r}: starting state differs from eager"
        e = rel_l2(out_g.float().cpu().numpy(), ref[r]["out"])
        es = rel_l2(st_g.cpu().numpy(), ref[r]["start_state"])
        assert e <= 1e-2 and es <= 1e-2, (r, e, es)
    B.raise_device_error(cr_g.workspace)
    assert all(torch.equal(x, y) for x, y in zip(cr_g.hist_len, cr_e.hist_len)) and torch.equal(cr_g.ckpt, cr_e.ckpt)


def test_bad_accepted_count_is_reported():
    from tree_forked_gated_amd import binding as B
    rng = np.random.default_rng(7)
    n_seq, N, H, D = 3, 4, 2, 64
    S0 = W._init(rng, n_seq, H, D, D, True)
    cr = B.ChainRounds(torch.from_numpy(S0).cuda(), N, 8, torch.float32, keep_state=True)
    f = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.float32)).cuda().contiguous()
    draft = {kk: f(x) for kk, x in _draft(rng, n_seq, N, H, D, "f32").items()}
    cr.step(draft, torch.zeros(n_seq, dtype=torch.int32, device="cuda"), check=True)
    cr.state.fill_(7.0)
    with pytest.raises(B.GdnDeviceError) as ei:
        cr.step(draft, torch.tensor([1, N + 1, 0], dtype=torch.int32, device="cuda"), check=True)
    assert ei.value.code == 9 and ei.value.index == 1
    assert bool((cr.state[1] == 7.0).all())  # the bad sequence is skipped
