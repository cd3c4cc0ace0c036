"""gdn_tree_forward_static, the forward for callers that cannot allocate: its
workspace is the library's static device array, not a caller buffer.

Two calls in a row (the second with a smaller stream and another structure,
so that it runs over the first call's leftover metadata) must give the same
bits as gdn_tree_forward with a workspace of its own, and match the oracle.
Sizes beyond the static array are refused on the host with a clear error."""
import numpy as np
import pytest
import torch

from tree_forked_gated_amd import workloads as W

from gpu_helpers import f64, oracle_ref, rel_l2, say, to_device, tol

pytestmark = pytest.mark.gpu


def _bits(t):
    return t.contiguous().view(torch.int16 if t.dtype == torch.bfloat16 else torch.int32)


def _run_both(wl):
    from tree_forked_gated_amd import binding as B
    d = to_device(wl)
    cap = B.capacities(wl.parent, wl.seq_start)
    rows = W.leaves_of(wl.parent)
    rows_d = torch.from_numpy(rows.astype(np.int32)).cuda()
    ref = B.forward(d["q"], d["k"], d["v"], d["log_gate"], d["beta"], d["parent_idx"], d["seq_start"],
                    d["init_state"], state_rows=rows_d, keep_pseudo=True, check=True, **cap)
    out = torch.full_like(ref.out, 3.0)
    st = torch.full_like(ref.state, 3.0)
    pv = torch.full_like(ref.pseudo_v, 3.0)
    B.forward_static(d["q"], d["k"], d["v"], d["log_gate"], d["beta"], d["parent_idx"], d["seq_start"],
                     d["init_state"], out=out, state_rows=rows_d, state_out=st, pseudo_v=pv, **cap)
    torch.cuda.synchronize()
    code, index = B.check_error(None)
    assert code == 0, (code, index)
    return ref, out, st, pv, rows


@pytest.mark.parametrize("dtype,D", [("bf16", 128), ("f32", 32)])
def test_static_forward_matches_forward_twice(dtype, D):
    big = W.random_small(501, n_seq=5, H=3, Dk=D, Dv=D, dtype=dtype, max_len=400)
    small = W.random_small(502, n_seq=2, H=3, Dk=D, Dv=D, dtype=dtype, max_len=150)
    assert small.T < big.T
    for name, wl in (("first", big), ("second, smaller", small)):
        say(f"static forward {dtype} D={D} {name}: T={wl.T} seqs={wl.n_seq}")
        ref, out, st, pv, rows = _run_both(wl)
        assert torch.equal(_bits(out), _bits(ref.out)), name
        assert torch.equal(_bits(st), _bits(ref.state)), name
        assert torch.equal(_bits(pv), _bits(ref.pseudo_v)), name
        o = oracle_ref(wl, state_rows=rows)
        errs = {"out": rel_l2(f64(out), o["out"]), "state": rel_l2(f64(st), o["state"]),
                "pseudo_v": rel_l2(f64(pv), o["pseudo_v"])}
        say(f"  rel-L2 vs oracle {errs}")
        assert all(e <= tol(wl) for e in errs.values()), errs


def test_static_forward_refuses_sizes_beyond_its_array():
    from tree_forked_gated_amd import binding as B
    # 40 fork slots x 32 heads x 64 KiB of fp32 state: 80 MiB, above the 64 MiB array
    dims = B.make_dims(4096, 32, 128, 128, 1, B.GDN_BF16, 40, 2)
    assert B.workspace_size(dims) > B.STATIC_WORKSPACE_BYTES
    e = lambda *s, dt=torch.bfloat16: torch.zeros(s, dtype=dt, device="cuda")
    q = e(4096, 32, 128)
    parent = torch.arange(-1, 4095, dtype=torch.int32, device="cuda")
    seq = torch.tensor([0, 4096], dtype=torch.int32, device="cuda")
    out = e(4096, 32, 128)
    with pytest.raises(B.GdnError, match="static workspace"):
        B.forward_static(q, q, q, e(4096, 32), e(4096, 32), parent, seq, None, out=out, max_forks=40, max_levels=2)
