"""The C-ABI library loads and exports what include/gdn_tree.h declares; host-only
calls and synchronous argument checks work without a GPU."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gdn_tree.h")


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(gdn_\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_boundary():
    names = _declared()
    for n in ["gdn_tree_forward", "gdn_tree_commit", "gdn_tree_workspace_size", "gdn_tree_check_error",
              "gdn_tree_strerror", "gdn_tree_plan", "gdn_tree_attention", "gdn_chain_step", "gdn_tree_forward_static"]:
        assert n in names


def test_library_exports_every_declared_symbol():
    from tree_forked_gated_amd import binding as B
    lib = ctypes.CDLL(B.LIB_PATH)
    missing = [n for n in _declared() if not hasattr(lib, n)]
    assert not missing, missing


def test_host_only_calls():
    from tree_forked_gated_amd import binding as B
    assert B.lib.gdn_tree_version() == 1
    d = B.make_dims(1000, 4, 128, 128, 3, B.GDN_BF16, 7, 3)
    n = B.workspace_size(d)
    L = B.plan_layout(d)
    assert L["total"] == n
    offs = [L[f] for f in B._LAYOUT_FIELDS if f != "total"]
    assert all(o % 256 == 0 for o in offs) and sorted(offs) == offs
    assert n - L["fork_states"] >= 7 * 4 * 128 * 128 * 4
    assert B.lib.gdn_tree_strerror(0) == b"ok"
    assert b"max_forks" in B.lib.gdn_tree_strerror(104)
    assert int(B.lib.gdn_tree_commit_workspace_size()) >= 8


@pytest.mark.parametrize("kw,code", [
    ({"dtype": 7}, -3),
    ({"Dk": 48}, -2),
    ({"Dk": 16, "dtype": 1}, -2),
    ({"Dk": 128, "dtype": 0}, -2),
    ({"Dv": 24}, -2),
    ({"Dv": 144}, -2),
    ({"H": 0}, -2),
    ({"max_levels": 0}, -2),
])
def test_bad_dims_are_rejected_on_the_host(kw, code):
    from tree_forked_gated_amd import binding as B
    base = dict(T=100, H=2, Dk=64, Dv=64, n_seq=1, dtype_code=B.GDN_BF16, max_forks=0, max_levels=1)
    if "dtype" in kw:
        base["dtype_code"] = kw.pop("dtype")
    base.update(kw)
    d = B.make_dims(**base)
    n = ctypes.c_size_t(0)
    assert B.lib.gdn_tree_workspace_size(ctypes.byref(d), ctypes.byref(n)) == code


def test_forward_argument_errors_need_no_gpu():
    from tree_forked_gated_amd import binding as B
    assert B.lib.gdn_tree_forward(None, None) == -1
    a = B.FwdArgs()
    a.dims = B.make_dims(100, 2, 64, 64, 1, B.GDN_BF16, 0, 1)
    assert B.lib.gdn_tree_forward(ctypes.byref(a), None) == -1  # no parent / seq_start / workspace
    a.parent_idx = a.seq_start = a.workspace = ctypes.c_void_p(4096)
    a.workspace_bytes = 16
    assert B.lib.gdn_tree_forward(ctypes.byref(a), None) == -4  # workspace too small
    a.workspace_bytes = 1 << 40
    assert B.lib.gdn_tree_forward(ctypes.byref(a), None) == -1  # q, k, v missing
    for f in ["q", "k", "v", "log_gate", "beta", "out"]:
        setattr(a, f, ctypes.c_void_p(8192))
    a.n_out = 5
    assert B.lib.gdn_tree_forward(ctypes.byref(a), None) == -6  # n_out must be T without out_rows
    a.n_out = 100
    a.dv_tile = 48
    assert B.lib.gdn_tree_forward(ctypes.byref(a), None) == -6
    a.dv_tile = 0
    a.q = ctypes.c_void_p(8194)
    assert B.lib.gdn_tree_forward(ctypes.byref(a), None) == -6  # misaligned
    assert b"aligned" in B.lib.gdn_tree_last_error()
    a.q = ctypes.c_void_p(8192)
    for f in ["out", "init_state", "pseudo_v"]:  # moved in 8- and 16-byte pieces
        setattr(a, f, ctypes.c_void_p(8200))
        assert B.lib.gdn_tree_forward(ctypes.byref(a), None) == -6, f
        assert b"aligned" in B.lib.gdn_tree_last_error()
        setattr(a, f, ctypes.c_void_p(8192) if f == "out" else None)


def test_capacities_match_reference_planner():
    from oracle import plan as P
    from tree_forked_gated_amd import binding as B
    from tree_forked_gated_amd import workloads as W
    for wl in [W.tiny_tree(), W.random_small(3, n_seq=6, max_len=300), W.mixed_forest(total=6000, H=1, D=32)]:
        ref = P.plan(wl.parent, wl.seq_start)
        cap = B.capacities(wl.parent, wl.seq_start)
        assert cap["max_forks"] == ref["n_fork"]
        assert cap["max_levels"] == max(1, ref["n_levels"])


@pytest.mark.parametrize("kw,code", [
    ({"dtype": 0}, -3),
    ({"D": 64}, -2),
    ({"Hq": 6, "Hkv": 4}, -2),
    ({"Hkv": 0}, -2),
    ({"max_levels": 0}, -2),
    ({"max_levels": 65}, -2),
    ({"T": -1}, -2),
])
def test_attention_bad_dims_are_rejected_on_the_host(kw, code):
    from tree_forked_gated_amd import binding as B
    base = dict(T=100, Hq=8, Hkv=2, D=128, n_seq=1, dtype=B.GDN_BF16, max_levels=4)
    base.update(kw)
    d = B.AttnDims(base["T"], base["Hq"], base["Hkv"], base["D"], base["n_seq"], base["dtype"], base["max_levels"])
    n = ctypes.c_size_t(0)
    assert B.lib.gdn_tree_attention_workspace_size(ctypes.byref(d), ctypes.byref(n)) == code


def test_attention_argument_errors_need_no_gpu():
    from tree_forked_gated_amd import binding as B
    assert B.lib.gdn_tree_attention(None, None) == -1
    d = B.attention_dims(100, 8, 2, 128, 1, 2)
    n = B.attention_workspace_size(d)
    assert n > 100 * (16 + 8 * 2)  # item and span tables on top of the planner's
    a = B.AttnArgs()
    a.dims = d
    a.scale = 0.1
    assert B.lib.gdn_tree_attention(ctypes.byref(a), None) == -1  # pointers missing
    for f in ["q", "k", "v", "out", "parent_idx", "seq_start", "workspace"]:
        setattr(a, f, ctypes.c_void_p(4096))
    a.workspace_bytes = 16
    assert B.lib.gdn_tree_attention(ctypes.byref(a), None) == -4  # workspace too small
    a.workspace_bytes = n
    a.k = ctypes.c_void_p(4100)
    assert B.lib.gdn_tree_attention(ctypes.byref(a), None) == -6  # misaligned
    a.k = ctypes.c_void_p(4096)
    a.flags = 2
    assert B.lib.gdn_tree_attention(ctypes.byref(a), None) == -6  # unknown flag
    a.flags = 0
    a.scale = float("nan")
    assert B.lib.gdn_tree_attention(ctypes.byref(a), None) == -6


def test_commit_argument_errors_need_no_gpu():
    """gdn_tree_commit refuses bad arguments on the host, before anything is
    enqueued: sizes, a negative path count, missing pointers and workspace,
    and states, keys or pseudo-values that are not 16-byte aligned."""
    from tree_forked_gated_amd import binding as B
    assert B.lib.gdn_tree_commit(None, None) == -1
    a = B.CommitArgs()
    a.dims = B.make_dims(100, 2, 48, 32, 1, B.GDN_BF16, 0, 1)
    assert B.lib.gdn_tree_commit(ctypes.byref(a), None) == -2  # d_k 48
    a.dims = B.make_dims(100, 2, 64, 32, 1, B.GDN_BF16, 0, 1)
    a.n_path = -1
    assert B.lib.gdn_tree_commit(ctypes.byref(a), None) == -6
    a.n_path = 3
    assert B.lib.gdn_tree_commit(ctypes.byref(a), None) == -1  # no workspace
    a.workspace = ctypes.c_void_p(4096)
    a.workspace_bytes = 4
    assert B.lib.gdn_tree_commit(ctypes.byref(a), None) == -4
    a.workspace_bytes = int(B.lib.gdn_tree_commit_workspace_size())
    assert B.lib.gdn_tree_commit(ctypes.byref(a), None) == -1  # k, paths, ... missing
    for f in ["k", "log_gate", "parent_idx", "seq_start", "init_state", "pseudo_v", "path_ptr", "path_nodes",
              "path_seq", "out_state"]:
        setattr(a, f, ctypes.c_void_p(8192))
    for f in ["out_state", "init_state", "k", "pseudo_v"]:
        setattr(a, f, ctypes.c_void_p(8200))
        assert B.lib.gdn_tree_commit(ctypes.byref(a), None) == -6, f
        assert b"aligned" in B.lib.gdn_tree_last_error()
        setattr(a, f, ctypes.c_void_p(8192))


def test_chain_argument_errors_need_no_gpu():
    """gdn_chain_step refuses bad arguments on the host, before anything is
    enqueued: sizes, missing buffers, buffers that must differ, misaligned
    rows, a too small workspace and unknown flags."""
    from tree_forked_gated_amd import binding as B
    assert B.lib.gdn_chain_step(None, None) == -1
    a = B.ChainArgs()
    for kw, code in [(dict(dtype=7), -3), (dict(N=0), -2), (dict(N=33), -2), (dict(Dk=16), -2), (dict(Dv=24), -2),
                     (dict(hist_cap=-1), -2)]:
        base = dict(n_seq=2, N=4, H=2, Dk=64, Dv=32, dtype=B.GDN_BF16, hist_cap=4)
        base.update(kw)
        a.dims = B.ChainDims(base["n_seq"], base["N"], base["H"], base["Dk"], base["Dv"], base["dtype"],
                             base["hist_cap"])
        assert B.lib.gdn_chain_step(ctypes.byref(a), None) == code, kw
    a.dims = B.ChainDims(2, 4, 2, 64, 32, B.GDN_BF16, 4)
    assert B.lib.gdn_chain_step(ctypes.byref(a), None) == -1  # buffers missing
    ptrs = ["ckpt", "hist_len_in", "hist_len_out", "prev_pv", "prev_k", "prev_g", "accepted", "q", "k", "v",
            "log_gate", "beta", "out", "pseudo_v", "workspace"]
    for i, f in enumerate(ptrs):
        setattr(a, f, ctypes.c_void_p(4096 * (i + 1)))
    assert B.lib.gdn_chain_step(ctypes.byref(a), None) == -1  # a history capacity needs the history buffers
    for i, f in enumerate(["hist_pv", "hist_k", "hist_g"]):
        setattr(a, f, ctypes.c_void_p(4096 * (len(ptrs) + i + 1)))
    a.hist_len_out = a.hist_len_in
    assert B.lib.gdn_chain_step(ctypes.byref(a), None) == -6
    a.hist_len_out = ctypes.c_void_p(4096 * 40)
    a.pseudo_v = a.prev_pv
    assert B.lib.gdn_chain_step(ctypes.byref(a), None) == -6
    a.pseudo_v = ctypes.c_void_p(4096 * 41)
    a.ckpt = ctypes.c_void_p(4096 + 8)
    assert B.lib.gdn_chain_step(ctypes.byref(a), None) == -6
    assert b"aligned" in B.lib.gdn_tree_last_error()
    a.ckpt = ctypes.c_void_p(4096)
    a.workspace_bytes = 4
    assert B.lib.gdn_chain_step(ctypes.byref(a), None) == -4
    a.workspace_bytes = 8
    a.flags = 4
    assert B.lib.gdn_chain_step(ctypes.byref(a), None) == -6  # unknown flag
