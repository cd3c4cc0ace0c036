"""ctypes binding of libgdn_tree.so (include/gdn_tree.h).

Argument marshalling only: every step of the forward and the commit runs in the
library's HIP kernels. PyTorch provides device memory and the current stream.
If the library has not been built, importing this module raises: there is no
fallback path.
"""
from __future__ import annotations

import contextlib
import ctypes
import gc
import os
from dataclasses import dataclass
from typing import Optional

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# GDN_TREE_LIB names another build of the same library (the stage-stamp
# measurement build, stage_stamps.py); by default the one beside this file.
LIB_PATH = os.environ.get("GDN_TREE_LIB") or os.path.join(_HERE, "libgdn_tree.so")

GDN_F32, GDN_BF16 = 0, 1
DEV_ERRORS = {0: "ok", 1: "seq_start", 2: "parent order", 3: "parent in another sequence", 4: "fork capacity",
              5: "level capacity", 6: "rows", 7: "commit path", 8: "workspace not planned for these sizes",
              9: "accepted count or history length out of range", 10: "cache_start"}
CHUNK = 64
FWD_PLANNED = 1  # gdn_tree.h GDN_FWD_PLANNED: reuse the metadata already in the workspace


class Dims(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int64), ("H", ctypes.c_int32), ("Dk", ctypes.c_int32), ("Dv", ctypes.c_int32),
                ("n_seq", ctypes.c_int32), ("dtype", ctypes.c_int32), ("max_forks", ctypes.c_int32),
                ("max_levels", ctypes.c_int32)]


class FwdArgs(ctypes.Structure):
    _fields_ = [("dims", Dims), ("q", ctypes.c_void_p), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
                ("log_gate", ctypes.c_void_p), ("beta", ctypes.c_void_p), ("parent_idx", ctypes.c_void_p),
                ("seq_start", ctypes.c_void_p), ("init_state", ctypes.c_void_p), ("out", ctypes.c_void_p),
                ("out_rows", ctypes.c_void_p), ("n_out", ctypes.c_int32), ("state_out", ctypes.c_void_p),
                ("state_rows", ctypes.c_void_p), ("n_state", ctypes.c_int32), ("pseudo_v", ctypes.c_void_p),
                ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t), ("dv_tile", ctypes.c_int32),
                ("flags", ctypes.c_uint32)]


class CommitArgs(ctypes.Structure):
    _fields_ = [("dims", Dims), ("k", ctypes.c_void_p), ("log_gate", ctypes.c_void_p),
                ("parent_idx", ctypes.c_void_p), ("seq_start", ctypes.c_void_p), ("init_state", ctypes.c_void_p),
                ("pseudo_v", ctypes.c_void_p), ("n_path", ctypes.c_int32), ("path_ptr", ctypes.c_void_p),
                ("path_nodes", ctypes.c_void_p), ("path_seq", ctypes.c_void_p), ("out_state", ctypes.c_void_p),
                ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t)]


class AttnDims(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int64), ("Hq", ctypes.c_int32), ("Hkv", ctypes.c_int32), ("D", ctypes.c_int32),
                ("n_seq", ctypes.c_int32), ("dtype", ctypes.c_int32), ("max_levels", ctypes.c_int32)]


class AttnArgs(ctypes.Structure):
    _fields_ = [("dims", AttnDims), ("scale", ctypes.c_float), ("q", ctypes.c_void_p), ("k", ctypes.c_void_p),
                ("v", ctypes.c_void_p), ("parent_idx", ctypes.c_void_p), ("seq_start", ctypes.c_void_p),
                ("out", ctypes.c_void_p), ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t),
                ("flags", ctypes.c_uint32), ("k_cache", ctypes.c_void_p), ("v_cache", ctypes.c_void_p),
                ("cache_start", ctypes.c_void_p), ("Tc", ctypes.c_int64)]


ATTN_PLANNED = 1  # gdn_tree.h GDN_ATTN_PLANNED

_LAYOUT_FIELDS = ["err", "n_seg", "n_fork", "tok_seq", "depth", "fork_slot", "seg_start", "seg_len", "seg_seq",
                  "seg_mode", "seg_entry", "seg_slot", "seg_level", "level_count", "level_ptr", "level_items",
                  "tree_mask", "fork_states", "total"]


class Layout(ctypes.Structure):
    _fields_ = [(f, ctypes.c_size_t) for f in _LAYOUT_FIELDS]


EXPORTS = ["gdn_tree_workspace_size", "gdn_tree_plan_layout", "gdn_tree_commit_workspace_size", "gdn_tree_plan",
           "gdn_tree_forward", "gdn_tree_forward_static", "gdn_tree_commit", "gdn_tree_check_error",
           "gdn_tree_strerror", "gdn_tree_last_error", "gdn_tree_version", "gdn_tree_attention_workspace_size",
           "gdn_tree_attention", "gdn_chain_step"]
STATIC_WORKSPACE_BYTES = 64 << 20  # gdn_tree.h GDN_TREE_STATIC_WORKSPACE_BYTES


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                          "(hipcc --offload-arch=gfx950); there is no fallback path")
    lib = ctypes.CDLL(LIB_PATH)
    for name in EXPORTS:
        getattr(lib, name)
    lib.gdn_tree_strerror.restype = ctypes.c_char_p
    lib.gdn_tree_last_error.restype = ctypes.c_char_p
    lib.gdn_tree_commit_workspace_size.restype = ctypes.c_size_t
    for name in ["gdn_tree_workspace_size", "gdn_tree_plan_layout", "gdn_tree_plan", "gdn_tree_forward",
                 "gdn_tree_forward_static", "gdn_tree_commit", "gdn_tree_check_error", "gdn_tree_version",
                 "gdn_tree_attention_workspace_size", "gdn_tree_attention", "gdn_chain_step"]:
        getattr(lib, name).restype = ctypes.c_int
    return lib


lib = _load()


class GdnError(RuntimeError):
    pass


class GdnDeviceError(GdnError):
    def __init__(self, code, index):
        super().__init__(f"device error {code} ({DEV_ERRORS.get(code, '?')}) at index {index}")
        self.code = code
        self.index = index


def _check(rc: int, what: str):
    if rc != 0:
        raise GdnError(f"{what}: {lib.gdn_tree_strerror(rc).decode()} ({rc}): {lib.gdn_tree_last_error().decode()}")


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _dtype_code(dt: torch.dtype) -> int:
    if dt == torch.float32:
        return GDN_F32
    if dt == torch.bfloat16:
        return GDN_BF16
    raise GdnError(f"unsupported dtype {dt}")


# ----------------------------------------------------------------- capacities

def capacities(parent, seq_start) -> dict:
    """Exact fork-slot and level counts of a tree whose structure is held on
    the host (numpy arrays or CPU tensors), from the same segment rules the
    device planner applies. An explicit utility: forward() never calls it, and
    it refuses device tensors rather than copy them back."""
    for x in (parent, seq_start):
        if isinstance(x, torch.Tensor) and x.device.type != "cpu":
            raise GdnError("capacities() takes a structure held on the host; pass the capacities of the "
                           "bucket instead of reading a device tree back")
    parent = np.asarray(parent, dtype=np.int64)
    seq_start = np.asarray(seq_start, dtype=np.int64)
    T = parent.shape[0]
    if T == 0:
        return {"max_forks": 0, "max_levels": 1}
    lens = np.diff(seq_start)
    tok_seq = np.repeat(np.arange(lens.shape[0]), lens)
    tree_tok = lens[tok_seq] <= CHUNK
    idx = np.arange(T)
    start = np.where(tree_tok, idx == seq_start[tok_seq], (parent < 0) | (parent != idx - 1))
    starts = np.nonzero(start)[0]
    entry = np.where(tree_tok[starts], -1, parent[starts])
    forks = np.unique(entry[entry >= 0])
    seg_of = np.cumsum(start) - 1
    level = np.zeros(starts.shape[0], dtype=np.int64)
    for i in np.nonzero(entry >= 0)[0]:
        level[i] = level[seg_of[entry[i]]] + 1
    return {"max_forks": int(forks.shape[0]), "max_levels": int(level.max()) + 1 if level.size else 1}


# ------------------------------------------------------------------- layouts

def make_dims(T, H, Dk, Dv, n_seq, dtype_code, max_forks, max_levels) -> Dims:
    return Dims(int(T), int(H), int(Dk), int(Dv), int(n_seq), int(dtype_code), int(max_forks), int(max_levels))


def workspace_size(dims: Dims) -> int:
    n = ctypes.c_size_t(0)
    _check(lib.gdn_tree_workspace_size(ctypes.byref(dims), ctypes.byref(n)), "gdn_tree_workspace_size")
    return int(n.value)


def plan_layout(dims: Dims) -> dict:
    L = Layout()
    _check(lib.gdn_tree_plan_layout(ctypes.byref(dims), ctypes.byref(L)), "gdn_tree_plan_layout")
    return {f: int(getattr(L, f)) for f in _LAYOUT_FIELDS}


def alloc_workspace(dims: Dims, device) -> torch.Tensor:
    return torch.empty(workspace_size(dims), dtype=torch.uint8, device=device)


def check_error(workspace: Optional[torch.Tensor], stream=None):
    """(code, index) of a workspace's error word; None reads the static
    workspace of forward_static on the current device."""
    code = ctypes.c_int32(0)
    index = ctypes.c_int64(0)
    _check(lib.gdn_tree_check_error(_ptr(workspace), _stream(stream), ctypes.byref(code), ctypes.byref(index)),
           "gdn_tree_check_error")
    return int(code.value), int(index.value)


def raise_device_error(workspace: torch.Tensor, stream=None):
    code, index = check_error(workspace, stream)
    if code != 0:
        raise GdnDeviceError(code, index)


# ------------------------------------------------------------------- forward

@dataclass
class ForwardResult:
    out: torch.Tensor
    state: torch.Tensor
    pseudo_v: Optional[torch.Tensor]
    workspace: torch.Tensor


def _fwd_args(q, k, v, log_gate, beta, parent_idx, seq_start, init_state, out, out_rows, state_out, state_rows,
              pseudo_v, workspace, dims, dv_tile, flags=0):
    a = FwdArgs()
    a.dims = dims
    a.q, a.k, a.v = _ptr(q), _ptr(k), _ptr(v)
    a.log_gate, a.beta = _ptr(log_gate), _ptr(beta)
    a.parent_idx, a.seq_start = _ptr(parent_idx), _ptr(seq_start)
    a.init_state = _ptr(init_state)
    a.out = _ptr(out) if out is not None and out.numel() > 0 else None
    a.out_rows = _ptr(out_rows)
    if out_rows is not None and out_rows.numel() == 0:
        # no readout rows: any valid address (never read) keeps "out_rows given" apart from "every token"
        a.out_rows = _ptr(parent_idx) if parent_idx is not None and parent_idx.numel() else _ptr(seq_start)
    a.n_out = int(out.shape[0]) if out is not None else 0
    a.state_out = _ptr(state_out) if state_out is not None and state_out.numel() > 0 else None
    a.state_rows = _ptr(state_rows) if state_rows is not None and state_rows.numel() > 0 else None
    a.n_state = int(state_rows.numel()) if state_rows is not None else 0
    a.pseudo_v = _ptr(pseudo_v)
    a.workspace = _ptr(workspace)
    a.workspace_bytes = 0 if workspace is None else int(workspace.numel())
    a.dv_tile = int(dv_tile)
    a.flags = int(flags)
    return a


def _i32(x, device):
    if x is None:
        return None
    if isinstance(x, torch.Tensor):
        return x.to(device=device, dtype=torch.int32).contiguous()
    return torch.as_tensor(np.asarray(x, dtype=np.int32), device=device)


def forward(q, k, v, log_gate, beta, parent_idx, seq_start, init_state=None, *, out_rows=None, state_rows=None,
            keep_pseudo=False, max_forks=None, max_levels=None, dv_tile=0, workspace=None, out=None, state_out=None,
            pseudo_v=None, stream=None, check=False, planned=False) -> ForwardResult:
    """gdn_tree_forward on torch tensors (device, contiguous).

    q, k [T,H,Dk], v [T,H,Dv], log_gate, beta [T,H] in float32 or bfloat16;
    parent_idx [T] and seq_start [n_seq+1] int32; init_state [n_seq,H,Dv,Dk]
    float32 or None. Returns out rows (all tokens unless out_rows), states of
    state_rows, pseudo-values when keep_pseudo, and the workspace (metadata and
    error word).

    max_forks and max_levels are the fork-slot and level capacities (Flide's
    fixed capacities per graph bucket, section 3.3.2); they are required. A
    tree that needs more raises a device error (see ``check``); nothing of the
    tree is read back to the host. planned=True reuses the metadata that an
    earlier call built in ``workspace`` for the same structure
    (GDN_FWD_PLANNED): only the walk runs."""
    if max_forks is None or max_levels is None:
        raise GdnError("forward() needs max_forks and max_levels (the bucket's capacities); "
                       "capacities() gives exact ones for a structure held on the host")
    device = q.device
    T, H, Dk = q.shape
    Dv = v.shape[2]
    parent_idx = _i32(parent_idx, device)
    seq_start = _i32(seq_start, device)
    out_rows = _i32(out_rows, device)
    state_rows = _i32(state_rows, device)
    n_seq = seq_start.numel() - 1
    dims = make_dims(T, H, Dk, Dv, n_seq, _dtype_code(q.dtype), max_forks, max(1, max_levels))
    if workspace is None:
        workspace = alloc_workspace(dims, device)
    n_out = T if out_rows is None else out_rows.numel()
    if out is None:
        out = torch.empty((n_out, H, Dv), dtype=q.dtype, device=device)
    n_state = 0 if state_rows is None else state_rows.numel()
    if state_out is None:
        state_out = torch.empty((n_state, H, Dv, Dk), dtype=torch.float32, device=device)
    if keep_pseudo and pseudo_v is None:
        pseudo_v = torch.empty((T, H, Dv), dtype=torch.float32, device=device)
    a = _fwd_args(q, k, v, log_gate, beta, parent_idx, seq_start, init_state, out, out_rows, state_out, state_rows,
                  pseudo_v, workspace, dims, dv_tile, FWD_PLANNED if planned else 0)
    _check(lib.gdn_tree_forward(ctypes.byref(a), _stream(stream)), "gdn_tree_forward")
    if check:
        raise_device_error(workspace, stream)
    return ForwardResult(out, state_out, pseudo_v, workspace)


def forward_static(q, k, v, log_gate, beta, parent_idx, seq_start, init_state, *, out, max_forks, max_levels,
                   out_rows=None, state_rows=None, state_out=None, pseudo_v=None, dv_tile=0, stream=None,
                   planned=False) -> None:
    """gdn_tree_forward_static: the forward with the library's static device
    workspace instead of a caller buffer. Every output buffer is the
    caller's (this wrapper allocates nothing either); errors are read with
    check_error(None)."""
    T, H, Dk = q.shape
    Dv = v.shape[2]
    n_seq = seq_start.numel() - 1
    dims = make_dims(T, H, Dk, Dv, n_seq, _dtype_code(q.dtype), max_forks, max(1, max_levels))
    a = _fwd_args(q, k, v, log_gate, beta, parent_idx, seq_start, init_state, out, out_rows, state_out, state_rows,
                  pseudo_v, None, dims, dv_tile, FWD_PLANNED if planned else 0)
    _check(lib.gdn_tree_forward_static(ctypes.byref(a), _stream(stream)), "gdn_tree_forward_static")


def plan(parent_idx, seq_start, *, T=None, H=1, Dk=16, Dv=16, dtype_code=GDN_F32, out_rows=None, state_rows=None,
         max_forks=None, max_levels=None, device="cuda", stream=None) -> dict:
    """Run only the metadata kernels and return every table (host numpy; an
    inspection utility that synchronises). Without capacities the structure
    must be given on the host, and its exact counts are used."""
    if max_forks is None or max_levels is None:
        try:
            cap = capacities(parent_idx, seq_start)
        except GdnError:
            raise
        except Exception:  # malformed structure: any capacity will do, the device reports the error
            n = int(np.asarray(parent_idx).shape[0])
            cap = {"max_forks": n, "max_levels": 8}
        max_forks = cap["max_forks"] if max_forks is None else max_forks
        max_levels = cap["max_levels"] if max_levels is None else max_levels
    parent_idx = _i32(parent_idx, device)
    seq_start = _i32(seq_start, device)
    out_rows = _i32(out_rows, device)
    state_rows = _i32(state_rows, device)
    T = parent_idx.numel() if T is None else T
    n_seq = seq_start.numel() - 1
    dims = make_dims(T, H, Dk, Dv, n_seq, dtype_code, max_forks, max(1, max_levels))
    ws = alloc_workspace(dims, device)
    a = FwdArgs()
    a.dims = dims
    a.parent_idx, a.seq_start = _ptr(parent_idx), _ptr(seq_start)
    a.out_rows = _ptr(out_rows)
    a.n_out = T if out_rows is None else out_rows.numel()
    a.state_rows = _ptr(state_rows)
    a.n_state = 0 if state_rows is None else state_rows.numel()
    a.workspace = _ptr(ws)
    a.workspace_bytes = ws.numel()
    _check(lib.gdn_tree_plan(ctypes.byref(a), _stream(stream)), "gdn_tree_plan")
    torch.cuda.synchronize(device)
    L = plan_layout(dims)
    host = ws.cpu().numpy()

    def i32(name, n):
        return host[L[name]:L[name] + 4 * n].view(np.int32).copy()

    word = int(host[L["err"]:L["err"] + 8].view(np.uint64)[0])
    err = (0, 0) if word == 0xFFFFFFFFFFFFFFFF else (word >> 32, word & 0xFFFFFFFF)
    n_seg = int(i32("n_seg", 1)[0])
    n_fork = int(i32("n_fork", 1)[0])
    ml = dims.max_levels
    out = {"error": err, "n_seg": n_seg, "n_fork": n_fork, "tok_seq": i32("tok_seq", T), "depth": i32("depth", T),
           "fork_slot": i32("fork_slot", T), "level_count": i32("level_count", ml),
           "level_ptr": i32("level_ptr", ml + 1),
           "tree_mask": host[L["tree_mask"]:L["tree_mask"] + 8 * n_seq * CHUNK].view(np.uint64).reshape(n_seq, CHUNK)
           .copy()}
    for f in ["seg_start", "seg_len", "seg_seq", "seg_mode", "seg_entry", "seg_slot", "seg_level", "level_items"]:
        out[f] = i32(f, T)[:n_seg]
    return out


# ----------------------------------------------------------------- attention

def attention_dims(T, Hq, Hkv, D, n_seq, max_levels) -> AttnDims:
    return AttnDims(int(T), int(Hq), int(Hkv), int(D), int(n_seq), GDN_BF16, int(max_levels))


def attention_workspace_size(dims: AttnDims) -> int:
    n = ctypes.c_size_t(0)
    _check(lib.gdn_tree_attention_workspace_size(ctypes.byref(dims), ctypes.byref(n)),
           "gdn_tree_attention_workspace_size")
    return int(n.value)


def attention(q, k, v, parent_idx, seq_start, *, max_levels, scale=None, workspace=None, out=None, planned=False,
              stream=None, check=False, k_cache=None, v_cache=None, cache_start=None):
    """gdn_tree_attention (ForkAttention) on device tensors: q [T,Hq,D], k and
    v [T,Hkv,D] bf16; returns (out [T,Hq,D], workspace). max_levels is the
    fork-nesting capacity (as for forward); scale defaults to 1/sqrt(D).
    k_cache, v_cache [Tc,Hkv,D] and cache_start [n_seq+1]: cached keys and
    values each sequence sees ahead of its tokens (optional)."""
    device = q.device
    T, Hq, D = q.shape
    Hkv = k.shape[1]
    parent_idx = _i32(parent_idx, device)
    seq_start = _i32(seq_start, device)
    dims = attention_dims(T, Hq, Hkv, D, seq_start.numel() - 1, max_levels)
    if workspace is None:
        workspace = torch.empty(attention_workspace_size(dims), dtype=torch.uint8, device=device)
    if out is None:
        out = torch.empty((T, Hq, D), dtype=q.dtype, device=device)
    a = AttnArgs()
    a.dims = dims
    a.scale = float(D ** -0.5 if scale is None else scale)
    a.q, a.k, a.v = _ptr(q), _ptr(k), _ptr(v)
    a.parent_idx, a.seq_start = _ptr(parent_idx), _ptr(seq_start)
    a.out = _ptr(out)
    a.workspace = _ptr(workspace)
    a.workspace_bytes = int(workspace.numel())
    a.flags = ATTN_PLANNED if planned else 0
    if cache_start is not None:
        cache_start = _i32(cache_start, device)
        a.cache_start = _ptr(cache_start)
        a.Tc = int(k_cache.shape[0])
        if a.Tc > 0:
            a.k_cache, a.v_cache = _ptr(k_cache), _ptr(v_cache)
    _check(lib.gdn_tree_attention(ctypes.byref(a), _stream(stream)), "gdn_tree_attention")
    if check:
        raise_device_error(workspace, stream)
    return out, workspace


# ------------------------------------------------------------- chain rounds

class ChainDims(ctypes.Structure):
    _fields_ = [("n_seq", ctypes.c_int32), ("N", ctypes.c_int32), ("H", ctypes.c_int32), ("Dk", ctypes.c_int32),
                ("Dv", ctypes.c_int32), ("dtype", ctypes.c_int32), ("hist_cap", ctypes.c_int32)]


class ChainArgs(ctypes.Structure):
    _fields_ = [("dims", ChainDims)] + [(f, ctypes.c_void_p) for f in (
        "ckpt", "hist_pv", "hist_k", "hist_g", "hist_len_in", "hist_len_out", "prev_pv", "prev_k", "prev_g",
        "accepted", "q", "k", "v", "log_gate", "beta", "out", "pseudo_v", "state_out", "workspace")] + [
        ("workspace_bytes", ctypes.c_size_t), ("flags", ctypes.c_uint32)]


CHAIN_FLUSH = 1  # gdn_tree.h GDN_CHAIN_FLUSH


class ChainRounds:
    """Device buffers of speculative chain rounds for n_seq sequences and
    gdn_chain_step over them (argument marshalling and buffer alternation only;
    the commit and the verify run in the library's kernel).

    ``step(draft, accepted)`` verifies a draft (dict of q, k, v, log_gate, beta
    tensors [n_seq, N, H, D], contiguous) after accepting ``accepted`` (device
    int32 [n_seq]) tokens of the previous draft, and returns (out, pseudo_v)
    views of the current draft buffers. The draft's k and log_gate tensors are
    the next step's prev_k and prev_g: keep them unchanged until then.
    ``state_out`` of the call receives the state each round starts from when
    ``keep_state`` is set."""

    def __init__(self, init_state, N, hist_cap, dtype, *, keep_state=False):
        dev = init_state.device
        n_seq, H, Dv, Dk = init_state.shape
        self.dims = ChainDims(n_seq, N, H, Dk, Dv, _dtype_code(dtype), hist_cap)
        self.ckpt = init_state.clone()
        cap = max(1, hist_cap)
        self.hist_pv = torch.zeros((n_seq, cap, H, Dv), dtype=torch.float32, device=dev)
        self.hist_k = torch.zeros((n_seq, cap, H, Dk), dtype=dtype, device=dev)
        self.hist_g = torch.zeros((n_seq, cap, H), dtype=torch.float32, device=dev)
        self.hist_len = [torch.zeros(n_seq, dtype=torch.int32, device=dev) for _ in range(2)]
        self.pv = [torch.zeros((n_seq, N, H, Dv), dtype=torch.float32, device=dev) for _ in range(2)]
        # the previous draft's keys and log gates (zeros before the first round)
        self.prev_k = torch.zeros((n_seq, N, H, Dk), dtype=dtype, device=dev)
        self.prev_g = torch.zeros((n_seq, N, H), dtype=dtype, device=dev)
        self.out = [torch.zeros((n_seq, N, H, Dv), dtype=dtype, device=dev) for _ in range(2)]
        self.state = torch.zeros_like(init_state) if keep_state else None
        self.workspace = torch.empty(int(lib.gdn_tree_commit_workspace_size()), dtype=torch.uint8, device=dev)
        self.cur = 0  # which draft buffers the next round writes

    def step(self, draft, accepted, *, flush=False, stream=None, check=False):
        c, p = self.cur, 1 - self.cur
        a = ChainArgs()
        a.dims = self.dims
        a.ckpt, a.hist_pv, a.hist_k, a.hist_g = _ptr(self.ckpt), _ptr(self.hist_pv), _ptr(self.hist_k), _ptr(self.hist_g)
        a.hist_len_in, a.hist_len_out = _ptr(self.hist_len[p]), _ptr(self.hist_len[c])
        a.prev_pv, a.prev_k, a.prev_g = _ptr(self.pv[p]), _ptr(self.prev_k), _ptr(self.prev_g)
        a.accepted = _ptr(accepted)
        a.q, a.k, a.v = _ptr(draft["q"]), _ptr(draft["k"]), _ptr(draft["v"])
        a.log_gate, a.beta = _ptr(draft["log_gate"]), _ptr(draft["beta"])
        a.out, a.pseudo_v = _ptr(self.out[c]), _ptr(self.pv[c])
        a.state_out = _ptr(self.state)
        a.workspace = _ptr(self.workspace)
        a.workspace_bytes = self.workspace.numel()
        a.flags = CHAIN_FLUSH if flush else 0
        _check(lib.gdn_chain_step(ctypes.byref(a), _stream(stream)), "gdn_chain_step")
        if check:
            raise_device_error(self.workspace, stream)
        self.prev_k, self.prev_g = draft["k"], draft["log_gate"]
        self.cur = p
        return self.out[c], self.pv[c]


# -------------------------------------------------------------------- commit

def commit(k, log_gate, parent_idx, seq_start, init_state, pseudo_v, path_ptr, path_nodes, path_seq, *,
           workspace=None, out_state=None, stream=None, check=False) -> torch.Tensor:
    """gdn_tree_commit: states after each accepted path (TreeWY Eq. 3)."""
    device = k.device
    T, H, Dk = k.shape
    Dv = pseudo_v.shape[2]
    parent_idx = _i32(parent_idx, device)
    seq_start = _i32(seq_start, device)
    path_ptr = _i32(path_ptr, device)
    path_nodes = _i32(path_nodes, device)
    path_seq = _i32(path_seq, device)
    n_path = path_ptr.numel() - 1
    if workspace is None:
        workspace = torch.empty(int(lib.gdn_tree_commit_workspace_size()), dtype=torch.uint8, device=device)
    if out_state is None:
        out_state = torch.empty((n_path, H, Dv, Dk), dtype=torch.float32, device=device)
    a = CommitArgs()
    a.dims = make_dims(T, H, Dk, Dv, seq_start.numel() - 1, _dtype_code(k.dtype), 0, 1)
    a.k, a.log_gate = _ptr(k), _ptr(log_gate)
    a.parent_idx, a.seq_start = _ptr(parent_idx), _ptr(seq_start)
    a.init_state, a.pseudo_v = _ptr(init_state), _ptr(pseudo_v)
    a.n_path = n_path
    a.path_ptr = _ptr(path_ptr)
    a.path_nodes = _ptr(path_nodes) if path_nodes.numel() else _ptr(path_ptr)
    a.path_seq = _ptr(path_seq)
    a.out_state = _ptr(out_state) if out_state.numel() else None
    a.workspace = _ptr(workspace)
    a.workspace_bytes = workspace.numel()
    _check(lib.gdn_tree_commit(ctypes.byref(a), _stream(stream)), "gdn_tree_commit")
    if check:
        raise_device_error(workspace, stream)
    return out_state


# -------------------------------------------------------------- graph replay

@contextlib.contextmanager
def capture_guard():
    """Python's cyclic garbage collector runs before a graph capture and stays
    off during it. A dead reference cycle that holds device tensors or graphs
    (an exception's traceback kept by a caller, say) would otherwise be
    finalised whenever the collector happens to run, and freeing or destroying
    device objects while a stream captures aborts the process."""
    gc.collect()
    was = gc.isenabled()
    gc.disable()
    try:
        yield
    finally:
        if was:
            gc.enable()


class ForwardGraph:
    """One captured forward (and optionally one commit) per size bucket,
    replayed for any tree that fits the bucket.

    Flide ("Accelerating Decision Inference with Exact State Forking", §3.3)
    captures a flat graph per stream-capacity bucket and replays it for every
    decision round. That works here because the tree is device data: the
    metadata kernels rebuild segments, fork slots, levels and masks from
    ``parent_idx`` inside the graph, and every launch shape depends only on
    the bucket (T, H, d_k, d_v, n_seq, the fork and level capacities, the
    numbers of output and state rows, and the number of commit paths), never
    on the tree. Levels beyond the tree's own are launched and exit at once.

    The buffers are static: ``load`` copies a round's tensors into them (with
    torch copies on the current stream, outside the graph), ``replay`` runs
    the captured kernels, and the results are read from ``out``, ``state_out``,
    ``pseudo_v`` and ``committed``. A tree that needs more fork slots or
    levels than the bucket holds is reported through the device error word
    (``check``), as in an eager call. The graph holds only kernel launches of
    this library (no memset nodes)."""

    def __init__(self, T, H, Dk, Dv, n_seq, dtype, *, max_forks, max_levels, n_out=None, n_state=0,
                 keep_pseudo=False, n_path=0, path_capacity=0, device="cuda"):
        dev = torch.device(device)
        self.device = dev
        self.dtype = dtype
        self.max_forks, self.max_levels = int(max_forks), max(1, int(max_levels))
        self.keep_pseudo = bool(keep_pseudo) or n_path > 0
        e = lambda *shape, dt=dtype: torch.zeros(shape, dtype=dt, device=dev)
        self.q, self.k = e(T, H, Dk), e(T, H, Dk)
        self.v = e(T, H, Dv)
        self.log_gate, self.beta = e(T, H), e(T, H)
        self.parent_idx = torch.full((T,), -1, dtype=torch.int32, device=dev)
        self.seq_start = torch.zeros(n_seq + 1, dtype=torch.int32, device=dev)
        self.init_state = e(n_seq, H, Dv, Dk, dt=torch.float32)
        self.out_rows = None if n_out is None else torch.zeros(n_out, dtype=torch.int32, device=dev)
        self.state_rows = torch.zeros(n_state, dtype=torch.int32, device=dev)
        self.out = e(T if n_out is None else n_out, H, Dv)
        self.state_out = e(n_state, H, Dv, Dk, dt=torch.float32)
        self.pseudo_v = e(T, H, Dv, dt=torch.float32) if self.keep_pseudo else None
        dims = make_dims(T, H, Dk, Dv, n_seq, _dtype_code(dtype), self.max_forks, self.max_levels)
        self.workspace = alloc_workspace(dims, dev)
        self.n_path = int(n_path)
        if self.n_path:
            self.path_ptr = torch.zeros(n_path + 1, dtype=torch.int32, device=dev)
            self.path_nodes = torch.zeros(max(1, int(path_capacity)), dtype=torch.int32, device=dev)
            self.path_seq = torch.zeros(n_path, dtype=torch.int32, device=dev)
            self.committed = e(n_path, H, Dv, Dk, dt=torch.float32)
            self.commit_workspace = torch.empty(int(lib.gdn_tree_commit_workspace_size()), dtype=torch.uint8,
                                                device=dev)
        self.graph = None

    def load(self, q, k, v, log_gate, beta, parent_idx, seq_start, init_state=None, *, out_rows=None,
             state_rows=None, path_ptr=None, path_nodes=None, path_seq=None):
        """Copy one round into the static buffers (shapes must match the bucket;
        path_nodes may be shorter than the path capacity)."""
        for dst, src in ((self.q, q), (self.k, k), (self.v, v), (self.log_gate, log_gate), (self.beta, beta)):
            dst.copy_(src)
        self.parent_idx.copy_(_i32(parent_idx, self.device))
        self.seq_start.copy_(_i32(seq_start, self.device))
        if init_state is None:
            self.init_state.zero_()
        else:
            self.init_state.copy_(init_state)
        if self.out_rows is not None:
            self.out_rows.copy_(_i32(out_rows, self.device))
        if self.state_rows.numel():
            self.state_rows.copy_(_i32(state_rows, self.device))
        if self.n_path:
            nodes = _i32(path_nodes, self.device)
            if nodes.numel() > self.path_nodes.numel():
                raise GdnError(f"{nodes.numel()} path nodes exceed the bucket's capacity {self.path_nodes.numel()}")
            self.path_ptr.copy_(_i32(path_ptr, self.device))
            self.path_nodes[:nodes.numel()].copy_(nodes)
            self.path_seq.copy_(_i32(path_seq, self.device))

    def _launch(self):
        forward(self.q, self.k, self.v, self.log_gate, self.beta, self.parent_idx, self.seq_start, self.init_state,
                out_rows=self.out_rows, state_rows=self.state_rows, keep_pseudo=self.keep_pseudo,
                max_forks=self.max_forks, max_levels=self.max_levels, workspace=self.workspace, out=self.out,
                state_out=self.state_out, pseudo_v=self.pseudo_v)
        if self.n_path:
            commit(self.k, self.log_gate, self.parent_idx, self.seq_start, self.init_state, self.pseudo_v,
                   self.path_ptr, self.path_nodes, self.path_seq, workspace=self.commit_workspace,
                   out_state=self.committed)

    def capture(self):
        """Capture the forward (and commit) on the loaded buffers. One eager run
        on a side stream comes first, so that nothing is initialised during
        capture."""
        s = torch.cuda.Stream(device=self.device)
        s.wait_stream(torch.cuda.current_stream(self.device))
        with torch.cuda.stream(s):
            self._launch()
        torch.cuda.current_stream(self.device).wait_stream(s)
        torch.cuda.synchronize(self.device)
        g = torch.cuda.CUDAGraph()
        with capture_guard(), torch.cuda.graph(g):
            self._launch()
        self.graph = g
        return self

    def replay(self):
        if self.graph is None:
            raise GdnError("ForwardGraph.replay before capture")
        self.graph.replay()

    def check(self, stream=None):
        """Raise the device error of the last replay, if any (synchronises)."""
        raise_device_error(self.workspace, stream)
        if self.n_path:
            raise_device_error(self.commit_workspace, stream)
