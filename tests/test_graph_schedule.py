"""Host logic of the graph family (Flide, "Accelerating Decision Inference
with Exact State Forking", section 3.3.2): smallest-fit bucket choice, splits
along request boundaries, requests that no bucket holds. No GPU needed: the
schedule reads only each request's structure."""
import numpy as np
import torch

from tree_forked_gated_amd.graphs import Bucket, GraphFamily, Request, request_needs


def _req(n, forks=(), out=1, state=0):
    """A chain of n tokens plus branches (fork token, length) appended after it."""
    par = list(range(-1, n - 1))
    for ft, bl in forks:
        b0 = len(par)
        par += [ft] + list(range(b0, b0 + bl - 1))
    par = np.array(par, np.int32)
    e = torch.empty(0)
    return Request(e, e, e, e, e, par, None, np.arange(len(par) - out, len(par), dtype=np.int32),
                   np.arange(state, dtype=np.int32))


FAM = GraphFamily([Bucket(4096, 8, 16, 3, 64, 32), Bucket(1024, 4, 8, 2, 16, 8)], 2, 128, 128, torch.bfloat16,
                  device="cpu")


def test_buckets_sorted_smallest_first():
    assert [b.T for b in FAM.buckets] == [1024, 4096]


def test_needs_count_forks_and_levels():
    r = _req(200, forks=[(100, 80), (150, 10)])
    nd = request_needs(r)
    assert (nd.tokens, nd.forks, nd.levels) == (290, 2, 2)
    nested = _req(200, forks=[(100, 80), (250, 90)])  # the second branch forks off the first
    assert request_needs(nested).levels == 3


def test_smallest_bucket_that_fits():
    assert FAM.schedule([_req(300), _req(400)]) == [(0, [0, 1])]
    # tokens fit the small bucket exactly: no filler sequence is needed
    assert FAM.schedule([_req(512), _req(512)]) == [(0, [0, 1])]
    # one token short: the filler takes a fifth sequence slot, more than the small bucket has
    assert FAM.schedule([_req(300)] * 4) == [(1, [0, 1, 2, 3])]
    # three fork levels need the large bucket
    assert FAM.schedule([_req(200, forks=[(100, 80), (250, 90)])]) == [(1, [0])]
    # readout rows beyond the small bucket's 16
    assert FAM.schedule([_req(100, out=20)]) == [(1, [0])]


def test_split_on_request_boundaries_and_oversize():
    reqs = [_req(1500), _req(1500), _req(1500), _req(5000), _req(200)]
    sched = FAM.schedule(reqs)
    assert sched == [(1, [0, 1]), (1, [2]), (None, [3]), (0, [4])]
    # every request is scheduled exactly once, in order
    assert [i for _, g in sched for i in g] == list(range(len(reqs)))


def test_spare_rows_are_distinct_and_unused():
    rows = GraphFamily._spare_rows(5, np.array([9, 8, 2]), 10, 8)
    assert sorted(rows.tolist()) == [3, 4, 5, 6, 7]
    rows = GraphFamily._spare_rows(3, np.array([0, 1]), 10, 6)
    assert rows.tolist() == [6, 7, 8]


def test_capture_guard_collects_first_and_keeps_the_collector_off():
    """A graph capture runs with Python's cyclic collector off, after one
    collection: a dead cycle is finalised before the capture, never inside it,
    and the collector's state is restored afterwards (also after an error)."""
    import gc

    from tree_forked_gated_amd import binding as B
    finalised = []

    class Holder:
        def __del__(self):
            finalised.append(gc.isenabled())

    a, b = Holder(), Holder()
    a.other, b.other = b, a  # a dead cycle once the names go
    del a, b
    assert gc.isenabled()
    with B.capture_guard():
        assert finalised == [True, True]  # collected at entry, before the body
        assert not gc.isenabled()
        c, d = Holder(), Holder()
        c.other, d.other = d, c
        del c, d
        for _ in range(2000):  # enough allocations to trip an automatic collection
            [object() for _ in range(10)]
        assert len(finalised) == 2
    assert gc.isenabled()
    gc.collect()
    assert len(finalised) == 4
    try:
        with B.capture_guard():
            raise ValueError("inside")
    except ValueError:
        pass
    assert gc.isenabled()
