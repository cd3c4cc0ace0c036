"""Flat graphs over stream lengths: a family of captured forwards, one per
capacity bucket, shared by every round whose packed stream fits (Flide,
"Accelerating Decision Inference with Exact State Forking", section 3.3.2
"Graphs over Stream Lengths").

Host-side runtime around the library; every step of the recurrence still runs
in its kernels. A round is a list of requests, each a small tree of tokens with
its own initial state (a decision request: a trunk and its question branches;
a draft tree; a resumed agent step). The scheduler that forms the round knows
each request's structure, so the capacities a round needs are counted on the
host from that structure; nothing is read back from the device.

* Buckets reserve fixed capacities: stream tokens T, sequences, fork-state
  slots, fork levels, readout rows and state rows. A round goes to the
  smallest bucket whose capacities hold it.
* Requests are packed without gaps, in order. The spare tokens at the tail
  form one filler sequence of zero-valued tokens (its own sequence, so no real
  token can reach it); empty sequences take the spare sequence slots, and the
  spare readout and state rows point at tokens nobody asked for.
* A round that no bucket holds is split along request boundaries into several
  replays; a single request larger than the largest bucket runs through the
  same library call without graph replay.

Every launch of a replay keeps the shape of its bucket; only buffer contents
change between rounds.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional, Sequence

import numpy as np
import torch

from . import binding as B


@dataclass(frozen=True)
class Bucket:
    """Fixed capacities of one captured graph."""
    T: int            # stream tokens
    n_seq: int        # sequences (requests plus the tail filler)
    max_forks: int    # fork-state slots
    max_levels: int   # fork levels
    n_out: int        # readout rows (at least 1)
    n_state: int      # state rows


@dataclass
class Request:
    """One request of a round. Tensors live on the device; the structure
    (local parents, readout and state rows) is the scheduler's host data."""
    q: torch.Tensor          # [n, H, Dk]
    k: torch.Tensor          # [n, H, Dk]
    v: torch.Tensor          # [n, H, Dv]
    log_gate: torch.Tensor   # [n, H]
    beta: torch.Tensor       # [n, H]
    parent: np.ndarray       # int32 [n]: local parent, -1 = the request's initial state
    init_state: Optional[torch.Tensor] = None  # [H, Dv, Dk] fp32, None = zeros
    out_rows: np.ndarray = field(default_factory=lambda: np.zeros(0, np.int32))    # local tokens read out
    state_rows: np.ndarray = field(default_factory=lambda: np.zeros(0, np.int32))  # local tokens whose state is kept

    @property
    def n(self) -> int:
        return int(self.parent.shape[0])


@dataclass
class RequestResult:
    out: torch.Tensor     # [len(out_rows), H, Dv]
    state: torch.Tensor   # [len(state_rows), H, Dv, Dk] fp32
    bucket: Optional[int]  # bucket index of the replay, None = run without a graph
    replay: int            # position of its replay (or eager run) within the round


@dataclass
class Needs:
    tokens: int
    forks: int
    levels: int
    out: int
    state: int


def request_needs(req: Request) -> Needs:
    """Capacities one request takes in a packed stream (fork slots and levels
    from the same segment rules as the device planner, on the request's own
    structure; both add up, respectively take the maximum, over requests)."""
    cap = B.capacities(req.parent, np.array([0, req.n], np.int64))
    return Needs(req.n, cap["max_forks"], cap["max_levels"], int(len(req.out_rows)), int(len(req.state_rows)))


class GraphFamily:
    """Captured forwards for a list of buckets (captured on first use)."""

    def __init__(self, buckets: Sequence[Bucket], H: int, Dk: int, Dv: int, dtype: torch.dtype,
                 device="cuda"):
        for b in buckets:
            if b.n_out < 1 or b.T < 1 or b.n_seq < 1 or b.max_levels < 1:
                raise B.GdnError(f"bucket {b}: T, n_seq, max_levels and n_out must be >= 1")
        self.buckets = sorted(buckets, key=lambda b: (b.T, b.n_seq, b.max_forks, b.max_levels, b.n_out, b.n_state))
        self.H, self.Dk, self.Dv, self.dtype = H, Dk, Dv, dtype
        self.device = torch.device(device)
        self.graphs: List[Optional[B.ForwardGraph]] = [None] * len(self.buckets)
        self.replays = [0] * len(self.buckets)  # replays served per bucket

    # ------------------------------------------------------------- scheduling

    def fits(self, bi: int, needs: Sequence[Needs]) -> bool:
        b = self.buckets[bi]
        tok = sum(x.tokens for x in needs)
        seqs = len(needs) + (1 if tok < b.T else 0)  # the tail filler is a sequence of its own
        return (tok <= b.T and seqs <= b.n_seq and sum(x.forks for x in needs) <= b.max_forks
                and max([x.levels for x in needs] + [1]) <= b.max_levels and sum(x.out for x in needs) <= b.n_out
                and sum(x.state for x in needs) <= b.n_state)

    def smallest(self, needs: Sequence[Needs]) -> Optional[int]:
        for bi in range(len(self.buckets)):
            if self.fits(bi, needs):
                return bi
        return None

    def schedule(self, requests: Sequence[Request]):
        """[(bucket index or None, [request indices])]: the whole round in the
        smallest bucket that holds it, else consecutive groups of requests
        that the largest bucket holds, each in its smallest bucket; a request
        that no bucket holds alone runs without a graph (None)."""
        needs = [request_needs(r) for r in requests]
        whole = self.smallest(needs)
        if whole is not None:
            return [(whole, list(range(len(requests))))]
        top = len(self.buckets) - 1
        groups, cur = [], []
        for i, nd in enumerate(needs):
            if not self.fits(top, [nd]):
                if cur:
                    groups.append(cur)
                    cur = []
                groups.append([i])
                continue
            if self.fits(top, [needs[j] for j in cur] + [nd]):
                cur.append(i)
            else:
                groups.append(cur)
                cur = [i]
        if cur:
            groups.append(cur)
        return [(self.smallest([needs[j] for j in g]), g) for g in groups]

    # ---------------------------------------------------------------- running

    def _graph(self, bi: int) -> B.ForwardGraph:
        if self.graphs[bi] is None:
            b = self.buckets[bi]
            self.graphs[bi] = B.ForwardGraph(b.T, self.H, self.Dk, self.Dv, b.n_seq, self.dtype,
                                             max_forks=b.max_forks, max_levels=b.max_levels, n_out=b.n_out,
                                             n_state=b.n_state, device=self.device)
        return self.graphs[bi]

    @staticmethod
    def _spare_rows(count: int, used: np.ndarray, T: int, filler0: int) -> np.ndarray:
        """`count` distinct tokens outside `used`: filler tokens first, then the
        stream's last tokens."""
        if count == 0:
            return np.zeros(0, np.int64)
        taken = np.zeros(T, bool)
        taken[used] = True
        order = np.concatenate([np.arange(filler0, T), np.arange(filler0 - 1, -1, -1)])
        free = order[~taken[order]]
        return free[:count]

    def _load(self, bi: int, reqs: Sequence[Request]):
        """Pack the requests into the bucket's static buffers; returns the row
        ranges of every request's readouts and states."""
        b = self.buckets[bi]
        fg = self._graph(bi)
        offs = np.cumsum([0] + [r.n for r in reqs])
        used = int(offs[-1])
        parent = np.empty(b.T, np.int64)
        seq_start = [0]
        out_rows, state_rows, out_rng, st_rng = [], [], [], []
        for r, o in zip(reqs, offs[:-1]):
            o = int(o)
            p = np.asarray(r.parent, np.int64)
            parent[o:o + r.n] = np.where(p < 0, -1, p + o)
            seq_start.append(o + r.n)
            out_rng.append((len(out_rows), len(out_rows) + len(r.out_rows)))
            st_rng.append((len(state_rows), len(state_rows) + len(r.state_rows)))
            out_rows += [int(x) + o for x in r.out_rows]
            state_rows += [int(x) + o for x in r.state_rows]
        if used < b.T:  # the tail filler: one chain of zero-valued tokens
            parent[used] = -1
            parent[used + 1:] = np.arange(used, b.T - 1)
            seq_start.append(b.T)
        seq_start += [b.T] * (b.n_seq + 1 - len(seq_start))
        out_rows = np.concatenate([np.asarray(out_rows, np.int64),
                                   self._spare_rows(b.n_out - len(out_rows), np.asarray(out_rows, np.int64), b.T,
                                                    used)])
        state_rows = np.concatenate([np.asarray(state_rows, np.int64),
                                     self._spare_rows(b.n_state - len(state_rows), np.asarray(state_rows, np.int64),
                                                      b.T, used)])
        for name in ("q", "k", "v", "log_gate", "beta"):
            dst = getattr(fg, name)
            for r, o in zip(reqs, offs[:-1]):
                dst[int(o):int(o) + r.n].copy_(getattr(r, name))
            if used < b.T:
                dst[used:].zero_()
        for i, r in enumerate(reqs):
            if r.init_state is None:
                fg.init_state[i].zero_()
            else:
                fg.init_state[i].copy_(r.init_state)
        if len(reqs) < b.n_seq:
            fg.init_state[len(reqs):].zero_()
        dev = self.device
        fg.parent_idx.copy_(torch.from_numpy(parent.astype(np.int32)).to(dev))
        fg.seq_start.copy_(torch.from_numpy(np.asarray(seq_start, np.int32)).to(dev))
        fg.out_rows.copy_(torch.from_numpy(out_rows.astype(np.int32)).to(dev))
        if b.n_state:
            fg.state_rows.copy_(torch.from_numpy(state_rows.astype(np.int32)).to(dev))
        return out_rng, st_rng

    def run(self, requests: Sequence[Request], check: bool = True) -> List[RequestResult]:
        """Run a round: one replay per scheduled group (eager for oversize
        requests). Results are copies, so the next replay may reuse the
        buffers. check=True reads each replay's device error word (a host
        synchronisation) and raises it."""
        results: List[Optional[RequestResult]] = [None] * len(requests)
        for pos, (bi, idx) in enumerate(self.schedule(requests)):
            reqs = [requests[i] for i in idx]
            if bi is None:
                r = reqs[0]
                nd = request_needs(r)
                res = B.forward(r.q, r.k, r.v, r.log_gate, r.beta, np.asarray(r.parent, np.int32),
                                np.array([0, r.n], np.int32),
                                None if r.init_state is None else r.init_state.unsqueeze(0).contiguous(),
                                out_rows=np.asarray(r.out_rows, np.int32),
                                state_rows=np.asarray(r.state_rows, np.int32), max_forks=nd.forks,
                                max_levels=nd.levels, check=check)
                results[idx[0]] = RequestResult(res.out, res.state, None, pos)
                continue
            out_rng, st_rng = self._load(bi, reqs)
            fg = self.graphs[bi]
            if fg.graph is None:
                fg.capture()
            else:
                fg.replay()
            self.replays[bi] += 1
            if check:
                fg.check()
            for i, (ro, rs) in zip(idx, zip(out_rng, st_rng)):
                results[i] = RequestResult(fg.out[ro[0]:ro[1]].clone(), fg.state_out[rs[0]:rs[1]].clone(), bi, pos)
        return results
