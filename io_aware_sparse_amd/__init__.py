"""Fused CSR neighbourhood attention for AMD MI355X (gfx950).

Thin Python binding over the C ABI in ``include/gnn_attn.h`` (library
``libgnn_attn.so`` built in-tree by ``python -m io_aware_sparse_amd.build``).
Every function here only marshals arguments: it checks shapes and dtypes,
allocates outputs with torch when the caller gives none, passes raw device
pointers and torch's current HIP stream, and turns a non-zero status into
:class:`GnnError`. All computation runs in the HIP library; there is no
fallback path, and calls fail loudly when the library is missing.

Function names match the C ABI: gnn_csr_build, gnn_plan_create,
gnn_plan_export, gnn_plan_destroy, gnn_attn_fwd, gnn_attn_fwd_noalloc, gnn_attn_bwd,
gatv2_attn_fwd, gatv2_attn_bwd, gnn_plan_set_timing, gnn_plan_timing_read,
gnn_build_checked, gnn_status_string.
"""
from __future__ import annotations

import ctypes as C
import os
from typing import Optional

_PKG = os.path.dirname(os.path.abspath(__file__))
# GNN_CHECKED=1 selects the checked build (graph validation in every call and
# device-side index checks; for debugging, not for speed)
LIB_PATH = os.path.join(_PKG, "libgnn_attn_checked.so" if os.environ.get("GNN_CHECKED") == "1" else "libgnn_attn.so")

GNN_F32, GNN_BF16 = 0, 1
GNN_OK = 0
STATUS = {0: "GNN_OK", -1: "GNN_ERR_INVALID_ARG", -2: "GNN_ERR_UNSUPPORTED", -3: "GNN_ERR_ALIGNMENT",
          -4: "GNN_ERR_OOM", -5: "GNN_ERR_HIP", -6: "GNN_ERR_BAD_GRAPH", -7: "GNN_ERR_SCRATCH"}

# exported symbols, in the order include/gnn_attn.h declares them
EXPORTS = ["gnn_plan_opts_default", "gnn_csr_build", "gnn_plan_create", "gnn_plan_export", "gnn_plan_destroy",
           "gnn_attn_fwd", "gnn_attn_fwd_noalloc", "gnn_attn_bwd", "gatv2_attn_fwd", "gatv2_attn_bwd", "gnn_plan_set_timing",
           "gnn_plan_timing_read", "gnn_status_string", "gnn_reduce_fwd", "gnn_reduce_bwd", "gnn_reorder",
           "gnn_permute_graph", "gnn_permute_rows", "gnn_spmm_prepare", "gnn_spmm", "gnn_build_checked"]
ORDERS = {"degree": 0, "rcm": 1}      # gnn_order_t
NORMS = {"sum": 0, "mean": 1, "gcn": 2}   # gnn_norm_t
REDUCE_OPS = {"max": 0, "min": 1}     # gnn_reduce_op_t
REDUCE_MSGS = {"src": 0, "diff": 1}   # gnn_msg_t


class GnnError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {STATUS.get(status, status)} ({gnn_status_string(status)})")


class PlanOpts(C.Structure):
    _fields_ = [("light_threshold", C.c_int32), ("chunk", C.c_int32), ("waves_per_group", C.c_int32),
                ("tile_density", C.c_float), ("want_csc", C.c_int32), ("sched_order", C.c_int32),
                ("xcd_split", C.c_int32)]


_P32 = C.POINTER(C.c_int32)


class PlanInfo(C.Structure):
    _fields_ = [("n_nodes", C.c_int32), ("n_edges", C.c_int64),
                ("light_threshold", C.c_int32), ("chunk", C.c_int32), ("waves_per_group", C.c_int32),
                ("n_light", C.c_int32), ("n_heavy", C.c_int32), ("n_groups", C.c_int32),
                ("light_ids", C.c_void_p), ("heavy_ids", C.c_void_p), ("groups", C.c_void_p),
                ("partial_ofs", C.c_void_p),
                ("has_csc", C.c_int32), ("cindptr", C.c_void_p), ("cindices", C.c_void_p),
                ("c_n_light", C.c_int32), ("c_n_heavy", C.c_int32), ("c_n_groups", C.c_int32),
                ("c_light_ids", C.c_void_p), ("c_heavy_ids", C.c_void_p), ("c_groups", C.c_void_p),
                ("c_partial_ofs", C.c_void_p),
                ("has_tiles", C.c_int32), ("n_tiles", C.c_int32), ("tile_min_nnz", C.c_int32),
                ("tile_rc", C.c_void_p), ("tile_mask", C.c_void_p), ("tile_ptr", C.c_void_p),
                ("rindptr", C.c_void_p), ("rindices", C.c_void_p), ("n_residual", C.c_int64),
                ("n_trb", C.c_int32), ("n_light_nt", C.c_int32), ("n_tcb", C.c_int32), ("n_c_light_nt", C.c_int32),
                ("trb", C.c_void_p), ("light_nt", C.c_void_p), ("ctile", C.c_void_p), ("ctile_ptr", C.c_void_p),
                ("tcb", C.c_void_p), ("rcindptr", C.c_void_p), ("rcindices", C.c_void_p),
                ("c_light_nt", C.c_void_p), ("light_sched", C.c_void_p), ("c_light_sched", C.c_void_p),
                ("structure_bytes", C.c_int64), ("workspace_bytes", C.c_int64),
                ("largest_workspace_alloc", C.c_int64), ("rows_sorted", C.c_int32),
                ("light_by_degree", C.c_void_p), ("c_light_by_degree", C.c_void_p), ("spmm_norm", C.c_int32),
                ("spmm_w", C.c_void_p), ("spmm_cw", C.c_void_p),
                ("n_long_light", C.c_int32), ("c_n_long_light", C.c_int32),
                ("n_xsplit_groups", C.c_int32), ("n_xsplit_slots", C.c_int32), ("xsplit_groups", C.c_void_p),
                ("xsplit_partial_ofs", C.c_void_p), ("xsplit_order", C.c_void_p)]


_lib = None


def lib():
    """The loaded HIP library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"HIP library missing: {LIB_PATH}; build it with "
                               "`python -m io_aware_sparse_amd.build`")
        # torch carries its own HIP runtime; load it first so that the library
        # binds to the same runtime instance (one HIP runtime per process)
        import torch  # noqa: F401
        L = C.CDLL(LIB_PATH)
        V, I32, I64, F = C.c_void_p, C.c_int32, C.c_int64, C.c_float
        L.gnn_plan_opts_default.argtypes = [C.POINTER(PlanOpts)]
        L.gnn_csr_build.argtypes = [V, V, I64, I32, I32, V, V, I64, C.POINTER(C.c_int64), V]
        L.gnn_plan_create.argtypes = [V, V, I32, I64, C.POINTER(PlanOpts), V, C.POINTER(V)]
        L.gnn_plan_export.argtypes = [V, C.POINTER(PlanInfo)]
        L.gnn_plan_destroy.argtypes = [V]
        L.gnn_attn_fwd.argtypes = [V, V, V, I32, I64, I32, I32, V, V, V, V, V, F, C.c_int, V]
        L.gnn_attn_fwd_noalloc.argtypes = [V, V, V, I32, I64, I32, I32, V, V, V, V, V, F, C.c_int, V]
        L.gnn_attn_bwd.argtypes = [V, V, V, I32, I64, I32, I32, V, V, V, V, V, V, V, V, V, F, C.c_int, V]
        L.gatv2_attn_fwd.argtypes = [V, V, V, I32, I64, I32, I32, V, V, V, V, F, V, V, C.c_int, V]
        L.gatv2_attn_bwd.argtypes = [V, V, V, I32, I64, I32, I32, V, V, V, V, F, V, V, V, V, V, V, C.c_int, V]
        L.gnn_reduce_fwd.argtypes = [V, V, V, I32, I64, I32, V, V, V, C.c_int, C.c_int, C.c_int, V]
        L.gnn_reduce_bwd.argtypes = [V, V, V, I32, I64, I32, V, V, V, C.c_int, C.c_int, V]
        L.gnn_reorder.argtypes = [V, V, I32, I64, C.c_int, V, V]
        L.gnn_permute_graph.argtypes = [V, V, I32, I64, V, V, V, V]
        L.gnn_permute_rows.argtypes = [V, V, I32, I64, V, I32, V]
        L.gnn_spmm_prepare.argtypes = [V, C.c_int, V]
        L.gnn_spmm.argtypes = [V, V, V, I32, I64, I32, V, V, I32, C.c_int, V]
        L.gnn_plan_set_timing.argtypes = [V, I32]
        L.gnn_plan_timing_read.argtypes = [V, I32, C.POINTER(C.c_char_p), C.POINTER(C.c_int32),
                                           C.POINTER(C.c_double), C.POINTER(C.c_int32)]
        L.gnn_build_checked.argtypes = []
        L.gnn_status_string.argtypes = [C.c_int]
        L.gnn_status_string.restype = C.c_char_p
        for name in EXPORTS:
            if name != "gnn_status_string":
                getattr(L, name).restype = C.c_int
        _lib = L
    return _lib


def gnn_status_string(status: int) -> str:
    return lib().gnn_status_string(int(status)).decode()


def _check(rc: int, where: str):
    if rc != GNN_OK:
        raise GnnError(rc, where)


def _torch():
    import torch
    return torch


def _stream(stream=None) -> int:
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream()
    return int(s.cuda_stream)


def _ptr(t) -> Optional[int]:
    return None if t is None else int(t.data_ptr())


def _fresh(t, stream=None):
    """An output buffer this binding allocated. They start uninitialised;
    with GNN_POISON_OUTPUTS=1 (a debugging aid) they start as NaN (integer
    outputs as INT32_MAX), filled on the call's stream, so that an element the
    library fails to write cannot pass for a plausible value."""
    if os.environ.get("GNN_POISON_OUTPUTS") == "1" and t.numel():
        torch = _torch()
        with torch.cuda.stream(stream if stream is not None else torch.cuda.current_stream()):
            t.fill_(float("nan") if t.is_floating_point() else 2 ** 31 - 1)
    return t


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.float32:
        return GNN_F32
    if t.dtype == torch.bfloat16:
        return GNN_BF16
    raise TypeError(f"features must be float32 or bfloat16, got {t.dtype}")


def _feat(t, name, shape=None, dtype=None):
    torch = _torch()
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a device tensor")
    if t.dim() != 3 or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous [N, H, D] tensor")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    return t


def _graph(indptr, indices):
    torch = _torch()
    for t, nm in ((indptr, "indptr"), (indices, "indices")):
        if not isinstance(t, torch.Tensor) or not t.is_cuda or t.dtype != torch.int32 or not t.is_contiguous():
            raise TypeError(f"{nm} must be a contiguous int32 device tensor")
    return int(indptr.numel()) - 1, int(indices.numel())


# ---------------------------------------------------------------------------

def gnn_csr_build(src, dst, n_nodes: int, add_self_loops: bool = True, stream=None):
    """CSR by destination (sorted, de-duplicated, optional self-loops) on the device.
    Returns (indptr int32 [N+1], indices int32 [E])."""
    torch = _torch()
    for t, nm in ((src, "src"), (dst, "dst")):
        if not t.is_cuda or t.dtype != torch.int32 or not t.is_contiguous():
            raise TypeError(f"{nm} must be a contiguous int32 device tensor")
    m = int(src.numel())
    if int(dst.numel()) != m:
        raise ValueError("src and dst differ in length")
    cap = m + (n_nodes if add_self_loops else 0)
    indptr = _fresh(torch.empty(n_nodes + 1, dtype=torch.int32, device=src.device), stream)
    indices = _fresh(torch.empty(max(cap, 1), dtype=torch.int32, device=src.device), stream)
    e = C.c_int64(0)
    _check(lib().gnn_csr_build(_ptr(src), _ptr(dst), m, int(n_nodes), int(bool(add_self_loops)), _ptr(indptr),
                               _ptr(indices), cap, C.byref(e), _stream(stream)), "gnn_csr_build")
    return indptr, indices[: e.value]


class Plan:
    """Owning handle of a gnn_plan_t; keeps the graph tensors alive."""

    def __init__(self, handle: int, indptr, indices, opts: PlanOpts):
        self.handle = handle
        self.indptr = indptr
        self.indices = indices
        self.opts = opts

    def __del__(self):
        h = getattr(self, "handle", None)
        if h and _lib is not None:
            _lib.gnn_plan_destroy(C.c_void_p(h))
            self.handle = None

    def destroy(self):
        if self.handle:
            lib().gnn_plan_destroy(C.c_void_p(self.handle))
            self.handle = None


def gnn_plan_create(indptr, indices, light_threshold: int = 512, chunk: int = 512, waves_per_group: int = 4,
                    tile_density: float = 0.0, want_csc: bool = False, sched_order: int = 2, xcd_split: bool = True,
                    stream=None) -> Plan:
    n, e = _graph(indptr, indices)
    o = PlanOpts()
    lib().gnn_plan_opts_default(C.byref(o))
    o.light_threshold, o.chunk, o.waves_per_group = int(light_threshold), int(chunk), int(waves_per_group)
    o.tile_density, o.want_csc, o.sched_order = float(tile_density), int(bool(want_csc)), int(sched_order)
    o.xcd_split = int(bool(xcd_split))
    h = C.c_void_p()
    _check(lib().gnn_plan_create(_ptr(indptr), _ptr(indices) if e else None, n, e, C.byref(o), _stream(stream),
                                 C.byref(h)), "gnn_plan_create")
    return Plan(h.value, indptr, indices, o)


def gnn_plan_destroy(plan: Plan):
    plan.destroy()


def _copy_dev(ptr, count, np_dtype):
    """Copy `count` elements from a device pointer to a new numpy array."""
    import numpy as np
    torch = _torch()
    out = np.empty(int(count), np_dtype)
    if count == 0 or not ptr:
        return out
    torch.cuda.synchronize()

    class _View:   # the plan's device array, seen by torch without a copy (torch reads it only)
        __cuda_array_interface__ = {"shape": (int(count),), "typestr": np.dtype(np_dtype).str,
                                    "data": (int(ptr), False), "version": 3}

    out[:] = torch.as_tensor(_View(), device="cuda").cpu().numpy()   # copied by torch's own HIP runtime
    return out


def gnn_plan_export(plan: Plan, arrays: bool = False) -> dict:
    """Plan counts (and, with arrays=True, host copies of its device arrays)."""
    import numpy as np
    info = PlanInfo()
    _check(lib().gnn_plan_export(C.c_void_p(plan.handle), C.byref(info)), "gnn_plan_export")
    d = {k: getattr(info, k) for k, t in PlanInfo._fields_ if t is not C.c_void_p}
    if arrays:
        n = info.n_nodes
        d["light"] = _copy_dev(info.light_ids, info.n_light, np.int32)
        d["heavy"] = _copy_dev(info.heavy_ids, info.n_heavy, np.int32)
        d["groups"] = _copy_dev(info.groups, 3 * info.n_groups, np.int32).reshape(-1, 3)
        d["partial_ofs"] = _copy_dev(info.partial_ofs, info.n_heavy + 1, np.int32)
        d["light_sched"] = _copy_dev(info.light_sched, info.n_light, np.int32)
        d["light_by_degree"] = _copy_dev(info.light_by_degree, info.n_light, np.int32)
        if info.has_csc:
            d["cindptr"] = _copy_dev(info.cindptr, n + 1, np.int32)
            d["cindices"] = _copy_dev(info.cindices, info.n_edges, np.int32)
            d["c_light"] = _copy_dev(info.c_light_ids, info.c_n_light, np.int32)
            d["c_heavy"] = _copy_dev(info.c_heavy_ids, info.c_n_heavy, np.int32)
            d["c_groups"] = _copy_dev(info.c_groups, 3 * info.c_n_groups, np.int32).reshape(-1, 3)
            d["c_partial_ofs"] = _copy_dev(info.c_partial_ofs, info.c_n_heavy + 1, np.int32)
            d["c_light_sched"] = _copy_dev(info.c_light_sched, info.c_n_light, np.int32)
            d["c_light_by_degree"] = _copy_dev(info.c_light_by_degree, info.c_n_light, np.int32)
        if info.n_xsplit_groups:
            d["xsplit_groups"] = _copy_dev(info.xsplit_groups, 3 * info.n_xsplit_groups, np.int32).reshape(-1, 3)
            d["xsplit_partial_ofs"] = _copy_dev(info.xsplit_partial_ofs, info.n_heavy + 1, np.int32)
            d["xsplit_order"] = _copy_dev(info.xsplit_order, info.n_xsplit_slots, np.int32)
        if info.spmm_w:
            d["spmm_w"] = _copy_dev(info.spmm_w, info.n_edges, np.float32)
        if info.spmm_cw:
            d["spmm_cw"] = _copy_dev(info.spmm_cw, info.n_edges, np.float32)
        if info.has_tiles:
            d["tile_rc"] = _copy_dev(info.tile_rc, 2 * info.n_tiles, np.int32).reshape(-1, 2)
            d["tile_mask"] = _copy_dev(info.tile_mask, 4 * info.n_tiles, np.uint64).reshape(-1, 4)
            d["tile_ptr"] = _copy_dev(info.tile_ptr, (n + 15) // 16 + 1, np.int32)
            d["rindptr"] = _copy_dev(info.rindptr, n + 1, np.int32)
            d["rindices"] = _copy_dev(info.rindices, info.n_residual, np.int32)
            d["trb"] = _copy_dev(info.trb, info.n_trb, np.int32)
            d["light_nt"] = _copy_dev(info.light_nt, info.n_light_nt, np.int32)
            d["ctile"] = _copy_dev(info.ctile, info.n_tiles, np.int32)
            d["ctile_ptr"] = _copy_dev(info.ctile_ptr, (n + 15) // 16 + 1, np.int32)
            if info.has_csc:
                d["tcb"] = _copy_dev(info.tcb, info.n_tcb, np.int32)
                d["rcindptr"] = _copy_dev(info.rcindptr, n + 1, np.int32)
                d["rcindices"] = _copy_dev(info.rcindices, info.n_residual, np.int32)
                d["c_light_nt"] = _copy_dev(info.c_light_nt, info.n_c_light_nt, np.int32)
    return d


def _plan_handle(plan):
    return None if plan is None else C.c_void_p(plan.handle)


def gnn_attn_fwd(plan: Optional[Plan], indptr, indices, Q, K, V, O=None, LSE=None, scale: float = 0.0,
                 want_lse: bool = True, stream=None):
    """Graph-Transformer attention forward. Returns (O, LSE or None)."""
    torch = _torch()
    n, e = _graph(indptr, indices)
    _feat(Q, "Q")
    N, H, D = Q.shape
    if N != n:
        raise ValueError("Q rows differ from the graph's node count")
    _feat(K, "K", Q.shape, Q.dtype)
    _feat(V, "V", Q.shape, Q.dtype)
    O = _fresh(torch.empty_like(Q), stream) if O is None else _feat(O, "O", Q.shape, Q.dtype)
    if LSE is None and want_lse:
        LSE = _fresh(torch.empty((N, H), dtype=torch.float32, device=Q.device), stream)
    _check(lib().gnn_attn_fwd(_plan_handle(plan), _ptr(indptr), _ptr(indices) if e else None, N, e, H, D,
                              _ptr(Q), _ptr(K), _ptr(V), _ptr(O), _ptr(LSE), float(scale), _dtype_code(Q),
                              _stream(stream)), "gnn_attn_fwd")
    return O, LSE


def gnn_attn_fwd_noalloc(plan: Optional[Plan], indptr, indices, Q, K, V, O, LSE=None, scale: float = 0.0,
                         stream=None):
    """Graph-Transformer attention forward through the entry point that
    allocates no device memory: O (and LSE, optional) must be given, and
    nothing is allocated here either. Returns (O, LSE)."""
    n, e = _graph(indptr, indices)
    _feat(Q, "Q")
    N, H, D = Q.shape
    if N != n:
        raise ValueError("Q rows differ from the graph's node count")
    _feat(K, "K", Q.shape, Q.dtype)
    _feat(V, "V", Q.shape, Q.dtype)
    _feat(O, "O", Q.shape, Q.dtype)
    if LSE is not None:
        torch = _torch()
        if not (LSE.is_cuda and LSE.dtype == torch.float32 and LSE.is_contiguous() and tuple(LSE.shape) == (N, H)):
            raise TypeError("LSE must be a contiguous float32 [N, H] device tensor")
    _check(lib().gnn_attn_fwd_noalloc(_plan_handle(plan), _ptr(indptr), _ptr(indices) if e else None, N, e, H, D,
                                      _ptr(Q), _ptr(K), _ptr(V), _ptr(O), _ptr(LSE), float(scale), _dtype_code(Q),
                                      _stream(stream)), "gnn_attn_fwd_noalloc")
    return O, LSE


def gatv2_attn_fwd(plan: Optional[Plan], indptr, indices, XD, XS, att, V=None, negative_slope: float = 0.2,
                   O=None, LSE=None, want_lse: bool = True, stream=None):
    """GATv2 attention forward (V defaults to XS itself). Returns (O, LSE or None)."""
    torch = _torch()
    n, e = _graph(indptr, indices)
    _feat(XD, "XD")
    N, H, D = XD.shape
    if N != n:
        raise ValueError("XD rows differ from the graph's node count")
    _feat(XS, "XS", XD.shape, XD.dtype)
    V = XS if V is None else _feat(V, "V", XD.shape, XD.dtype)
    if not (att.is_cuda and att.dtype == torch.float32 and att.is_contiguous() and tuple(att.shape) == (H, D)):
        raise TypeError("att must be a contiguous float32 [H, D] device tensor")
    O = _fresh(torch.empty_like(XD), stream) if O is None else _feat(O, "O", XD.shape, XD.dtype)
    if LSE is None and want_lse:
        LSE = _fresh(torch.empty((N, H), dtype=torch.float32, device=XD.device), stream)
    _check(lib().gatv2_attn_fwd(_plan_handle(plan), _ptr(indptr), _ptr(indices) if e else None, N, e, H, D,
                                _ptr(XD), _ptr(XS), _ptr(V), _ptr(att), float(negative_slope), _ptr(O), _ptr(LSE),
                                _dtype_code(XD), _stream(stream)), "gatv2_attn_fwd")
    return O, LSE


def gnn_attn_bwd(plan: Plan, indptr, indices, Q, K, V, O, dO, LSE, dQ=None, dK=None, dV=None, scale: float = 0.0,
                 stream=None):
    """Graph-Transformer attention backward from the cached LSE. Returns (dQ, dK, dV)."""
    torch = _torch()
    n, e = _graph(indptr, indices)
    _feat(Q, "Q")
    N, H, D = Q.shape
    for t, nm in ((K, "K"), (V, "V"), (dO, "dO")):
        _feat(t, nm, Q.shape, Q.dtype)
    if O is not None:
        _feat(O, "O", Q.shape, Q.dtype)
    if not (LSE.is_cuda and LSE.dtype == torch.float32 and tuple(LSE.shape) == (N, H) and LSE.is_contiguous()):
        raise TypeError("LSE must be a contiguous float32 [N, H] device tensor")
    dQ = _fresh(torch.empty_like(Q), stream) if dQ is None else _feat(dQ, "dQ", Q.shape, Q.dtype)
    dK = _fresh(torch.empty_like(Q), stream) if dK is None else _feat(dK, "dK", Q.shape, Q.dtype)
    dV = _fresh(torch.empty_like(Q), stream) if dV is None else _feat(dV, "dV", Q.shape, Q.dtype)
    _check(lib().gnn_attn_bwd(_plan_handle(plan), _ptr(indptr), _ptr(indices) if e else None, N, e, H, D,
                              _ptr(Q), _ptr(K), _ptr(V), _ptr(O), _ptr(dO), _ptr(LSE), _ptr(dQ), _ptr(dK), _ptr(dV),
                              float(scale), _dtype_code(Q), _stream(stream)), "gnn_attn_bwd")
    return dQ, dK, dV


def gatv2_attn_bwd(plan: Plan, indptr, indices, XD, XS, att, dO, LSE, V=None, negative_slope: float = 0.2,
                   dXD=None, dXS=None, dV=None, d_att=None, stream=None):
    """GATv2 attention backward from the cached LSE. Returns (dXD, dXS, dV or
    None, d_att); with V None (V is XS) dXS includes the value gradient."""
    torch = _torch()
    n, e = _graph(indptr, indices)
    _feat(XD, "XD")
    N, H, D = XD.shape
    _feat(XS, "XS", XD.shape, XD.dtype)
    _feat(dO, "dO", XD.shape, XD.dtype)
    sep = V is not None and V.data_ptr() != XS.data_ptr()
    Vt = _feat(V, "V", XD.shape, XD.dtype) if sep else XS
    if not (att.is_cuda and att.dtype == torch.float32 and att.is_contiguous() and tuple(att.shape) == (H, D)):
        raise TypeError("att must be a contiguous float32 [H, D] device tensor")
    if not (LSE.is_cuda and LSE.dtype == torch.float32 and tuple(LSE.shape) == (N, H) and LSE.is_contiguous()):
        raise TypeError("LSE must be a contiguous float32 [N, H] device tensor")
    dXD = _fresh(torch.empty_like(XD), stream) if dXD is None else _feat(dXD, "dXD", XD.shape, XD.dtype)
    dXS = _fresh(torch.empty_like(XD), stream) if dXS is None else _feat(dXS, "dXS", XD.shape, XD.dtype)
    if sep:
        dV = _fresh(torch.empty_like(XD), stream) if dV is None else _feat(dV, "dV", XD.shape, XD.dtype)
    else:
        dV = None
    d_att = _fresh(torch.empty((H, D), dtype=torch.float32, device=XD.device), stream) if d_att is None else d_att
    _check(lib().gatv2_attn_bwd(_plan_handle(plan), _ptr(indptr), _ptr(indices) if e else None, N, e, H, D,
                                _ptr(XD), _ptr(XS), _ptr(Vt), _ptr(att), float(negative_slope), _ptr(dO), _ptr(LSE),
                                _ptr(dXD), _ptr(dXS), _ptr(dV), _ptr(d_att), _dtype_code(XD), _stream(stream)),
           "gatv2_attn_bwd")
    return dXD, dXS, dV, d_att


def gnn_build_checked() -> bool:
    """True when the loaded library is the checked build."""
    return bool(lib().gnn_build_checked())


def gnn_plan_set_timing(plan: Plan, enable: bool = True):
    _check(lib().gnn_plan_set_timing(C.c_void_p(plan.handle), int(bool(enable))), "gnn_plan_set_timing")


def _rows2d(t, name, shape=None, dtype=None):
    torch = _torch()
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a device tensor")
    if t.dim() != 2 or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous [N, F] tensor")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    return t


def gnn_reduce_fwd(plan: Optional[Plan], indptr, indices, X, op: str = "max", msg: str = "src", out=None,
                   arg=None, want_arg: bool = True, stream=None):
    """Neighbourhood max / min of per-edge messages (X[j], or X[j] - X[i] for
    msg "diff") with the smallest winning source. X is [N, F] float32 or
    bfloat16. Returns (out, arg int32 or None)."""
    torch = _torch()
    n, e = _graph(indptr, indices)
    _rows2d(X, "X")
    _dtype_code(X)
    N, F = X.shape
    if N != n:
        raise ValueError("X rows differ from the graph's node count")
    out = _fresh(torch.empty_like(X), stream) if out is None else _rows2d(out, "out", X.shape, X.dtype)
    if arg is None and want_arg:
        arg = _fresh(torch.empty((N, F), dtype=torch.int32, device=X.device), stream)
    elif arg is not None:
        _rows2d(arg, "arg", X.shape, torch.int32)
    _check(lib().gnn_reduce_fwd(_plan_handle(plan), _ptr(indptr), _ptr(indices) if e else None, N, e, F, _ptr(X),
                                _ptr(out), _ptr(arg), REDUCE_OPS[op], REDUCE_MSGS[msg], _dtype_code(X),
                                _stream(stream)), "gnn_reduce_fwd")
    return out, arg


def gnn_reduce_bwd(plan: Plan, indptr, indices, dOut, arg, msg: str = "src", dX=None, stream=None):
    """Gradient of gnn_reduce_fwd through its winners `arg`. Returns dX."""
    torch = _torch()
    n, e = _graph(indptr, indices)
    _rows2d(dOut, "dOut")
    _dtype_code(dOut)
    N, F = dOut.shape
    if N != n:
        raise ValueError("dOut rows differ from the graph's node count")
    _rows2d(arg, "arg", dOut.shape, torch.int32)
    dX = _fresh(torch.empty_like(dOut), stream) if dX is None else _rows2d(dX, "dX", dOut.shape, dOut.dtype)
    _check(lib().gnn_reduce_bwd(_plan_handle(plan), _ptr(indptr), _ptr(indices) if e else None, N, e, F, _ptr(dOut),
                                _ptr(arg), _ptr(dX), REDUCE_MSGS[msg], _dtype_code(dOut), _stream(stream)),
           "gnn_reduce_bwd")
    return dX


def gnn_spmm_prepare(plan: Plan, norm: str = "gcn", stream=None) -> None:
    """Cache the SpMM weights of `norm` ("sum", "mean", "gcn") in the plan."""
    _check(lib().gnn_spmm_prepare(C.c_void_p(plan.handle), NORMS[norm], _stream(stream)), "gnn_spmm_prepare")


def gnn_spmm(plan: Plan, indptr, indices, X, transpose: bool = False, Y=None, stream=None):
    """Y = A_w X (or A_w^T X) with the plan's cached weights; X [N, F]."""
    torch = _torch()
    n, e = _graph(indptr, indices)
    _rows2d(X, "X")
    _dtype_code(X)
    N, F = X.shape
    if N != n:
        raise ValueError("X rows differ from the graph's node count")
    Y = _fresh(torch.empty_like(X), stream) if Y is None else _rows2d(Y, "Y", X.shape, X.dtype)
    _check(lib().gnn_spmm(_plan_handle(plan), _ptr(indptr), _ptr(indices) if e else None, N, e, F, _ptr(X), _ptr(Y),
                          int(bool(transpose)), _dtype_code(X), _stream(stream)), "gnn_spmm")
    return Y


def gnn_reorder(indptr, indices, method: str = "rcm", stream=None):
    """Node order for relabelling (perm[new] = old, int32 device tensor)."""
    torch = _torch()
    n, e = _graph(indptr, indices)
    perm = _fresh(torch.empty(max(n, 0), dtype=torch.int32, device=indptr.device), stream)
    _check(lib().gnn_reorder(_ptr(indptr), _ptr(indices) if e else None, n, e, ORDERS[method], _ptr(perm),
                             _stream(stream)), "gnn_reorder")
    return perm


def gnn_permute_graph(indptr, indices, perm, stream=None):
    """CSR of the graph relabelled by perm (new row r = old row perm[r], rows sorted)."""
    torch = _torch()
    n, e = _graph(indptr, indices)
    if perm.dtype != torch.int32 or not perm.is_cuda or perm.numel() != n or not perm.is_contiguous():
        raise TypeError("perm must be a contiguous int32 device tensor of N entries")
    nip = _fresh(torch.empty_like(indptr), stream)
    nix = _fresh(torch.empty_like(indices), stream)
    _check(lib().gnn_permute_graph(_ptr(indptr), _ptr(indices) if e else None, n, e, _ptr(perm), _ptr(nip),
                                   _ptr(nix) if e else None, _stream(stream)), "gnn_permute_graph")
    return nip, nix


def gnn_permute_rows(src, perm, back: bool = False, dst=None, stream=None):
    """Rows of src (first dimension = nodes) in the new order (dst[r] = src[perm[r]]),
    or back to the old order (dst[perm[r]] = src[r])."""
    torch = _torch()
    if not src.is_cuda or not src.is_contiguous():
        raise TypeError("src must be a contiguous device tensor")
    n = src.shape[0]
    if perm.dtype != torch.int32 or perm.numel() != n or not perm.is_contiguous():
        raise TypeError("perm must be a contiguous int32 tensor of src.shape[0] entries")
    dst = _fresh(torch.empty_like(src), stream) if dst is None else dst
    row_bytes = src[0].numel() * src.element_size() if n else 0
    _check(lib().gnn_permute_rows(_ptr(src), _ptr(dst), n, row_bytes, _ptr(perm), int(bool(back)), _stream(stream)),
           "gnn_permute_rows")
    return dst


def gnn_plan_timing_read(plan: Plan) -> dict:
    """{kernel name: (launches, total ms)} since the last read; clears the log."""
    cap = 64
    names = (C.c_char_p * cap)()
    launches = (C.c_int32 * cap)()
    ms = (C.c_double * cap)()
    n = C.c_int32(0)
    _check(lib().gnn_plan_timing_read(C.c_void_p(plan.handle), cap, names, launches, ms, C.byref(n)),
           "gnn_plan_timing_read")
    return {names[k].decode(): (int(launches[k]), float(ms[k])) for k in range(min(n.value, cap))}
