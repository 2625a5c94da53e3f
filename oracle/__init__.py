"""Reference oracle for fused CSR neighbourhood attention.

TEST INFRASTRUCTURE ONLY: only ``tests/``, the smoke check and the benchmark's
CPU-baseline leg may import this package. The HIP library never imports,
links or calls it, and it imports nothing from the library.

Two halves:

* integer structure (plain numpy, exact): CSR by destination, degree
  bucketing into light/heavy nodes with the heavy chunk table, the transposed
  adjacency (CSC), and the 16x16 dense-tile census. These are the definitions
  the preprocessor must reproduce bit for bit.
* floating point (``oracle.c``, fp64, OpenMP over rows): Graph-Transformer
  forward and backward and GATv2 forward and backward, each materialising
  per-row edge logits and using a two-pass softmax; the neighbourhood
  max/min reduction with its winning indices (decided in fp32, the
  messages' precision) and its gradient.

Source: "On Efficient Scaling of GNNs via IO-Aware Layers Implementations",
technical summary, Methodology (degree-aware tiling with a light/heavy split;
fused CSR attention with an online-softmax forward and a log-sum-exp
recompute backward; reduction-based aggregations (a per-edge computation and
a neighbourhood min/max); cached transposed adjacency; 16x16 block-sparse
tiles).
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")


def build(force: bool = True) -> str:
    """Compile oracle.c with gcc (fp64, no fast-math) into liboracle.so."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-fno-fast-math",
               "-ffp-contract=off", "-Wall", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=False)
        lib = C.CDLL(_LIB)
        P = C.c_void_p
        i64, i32, f64 = C.c_int64, C.c_int, C.c_double
        lib.orc_gt_fwd.argtypes = [i64, P, P, i32, i32, P, P, P, f64, i64, P, P, P, P, P]
        lib.orc_gatv2_fwd.argtypes = [i64, P, P, i32, i32, P, P, P, P, f64, i64, P, P, P, P, P]
        lib.orc_gt_bwd_rows.argtypes = [i64, P, P, i32, i32, P, P, P, P, f64, i64, P, P, P, P, P, P]
        lib.orc_gt_bwd_srcs.argtypes = [i64, P, P, i32, i32, P, P, P, P, f64, P, P, P, P, i64, P, P, P, P, P]
        lib.orc_gatv2_bwd_rows.argtypes = [i64, P, P, i32, i32, P, P, P, P, f64, P, i64, P, P, P, P, P, P, P, P]
        lib.orc_gatv2_bwd_srcs.argtypes = [i64, P, P, i32, i32, P, P, P, P, f64, P, P, P, P, P, i64, P, P, P, P, P]
        lib.orc_segment_reduce.argtypes = [i64, P, P, i64, P, i32, i32, i64, P, P, P]
        for f in (lib.orc_gt_fwd, lib.orc_gatv2_fwd, lib.orc_gt_bwd_rows, lib.orc_gt_bwd_srcs, lib.orc_gatv2_bwd_rows,
                  lib.orc_gatv2_bwd_srcs, lib.orc_segment_reduce):
            f.restype = C.c_int
        lib.orc_num_threads.restype = C.c_int
        _lib = lib
    return _lib


def num_threads() -> int:
    return int(_load().orc_num_threads())


def set_threads(n: int) -> None:
    """Use n OpenMP threads in later calls (results do not depend on it:
    each output row is reduced by one thread in a fixed order)."""
    L = _load()
    L.orc_set_threads.argtypes = [C.c_int]
    L.orc_set_threads(int(n))


def _p(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


def _f64(x) -> np.ndarray:
    return np.ascontiguousarray(x, dtype=np.float64)


# ---------------------------------------------------------------------------
# integer structure
# ---------------------------------------------------------------------------

def csr_build(src, dst, n_nodes: int, add_self_loops: bool = True):
    """CSR by destination from a COO edge list (edge src -> dst).

    Row i holds the sources of i's in-edges in ascending order; duplicate
    pairs are removed; with add_self_loops, (i, i) is present exactly once in
    every row. Returns (indptr int32 [N+1], indices int32 [E])."""
    n = int(n_nodes)
    s = np.asarray(src, np.int64).ravel()
    d = np.asarray(dst, np.int64).ravel()
    if s.size and (s.min() < 0 or s.max() >= n or d.min() < 0 or d.max() >= n):
        raise ValueError("edge endpoint out of range")
    if add_self_loops:
        s = np.concatenate([s, np.arange(n, dtype=np.int64)])
        d = np.concatenate([d, np.arange(n, dtype=np.int64)])
    keys = np.unique(d * n + s)
    rows = keys // n
    indices = (keys - rows * n).astype(np.int32)
    indptr = np.zeros(n + 1, np.int64)
    np.cumsum(np.bincount(rows, minlength=n), out=indptr[1:])
    return indptr.astype(np.int32), indices


def degrees(indptr) -> np.ndarray:
    return np.diff(np.asarray(indptr, np.int64))


def bucketing(indptr, threshold: int, chunk: int, waves: int):
    """Degree-aware light/heavy split and heavy chunk-group table.

    light = nodes with degree <= threshold, heavy = the rest, each ascending.
    Each heavy node's edge range is cut into groups of chunk*waves edges (the
    last may be short); a group is one workgroup whose waves each take one
    chunk of <= chunk edges. partial_ofs[k]..partial_ofs[k+1] are the groups
    (and partial-result slots) of heavy node k.

    Returns dict: light int32 [n_light], heavy int32 [n_heavy],
    groups int32 [n_groups, 3] = (node, e0, e1), partial_ofs int32 [n_heavy+1]."""
    ip = np.asarray(indptr, np.int64)
    deg = np.diff(ip)
    light = np.nonzero(deg <= threshold)[0]
    heavy = np.nonzero(deg > threshold)[0]
    span = int(chunk) * int(waves)
    ng = (deg[heavy] + span - 1) // span
    partial_ofs = np.zeros(heavy.size + 1, np.int64)
    np.cumsum(ng, out=partial_ofs[1:])
    node = np.repeat(heavy, ng)
    k = np.arange(node.size) - np.repeat(partial_ofs[:-1], ng)
    e0 = ip[node] + k * span
    e1 = np.minimum(e0 + span, ip[node + 1])
    groups = np.stack([node, e0, e1], axis=1) if node.size else np.zeros((0, 3), np.int64)
    return dict(light=light.astype(np.int32), heavy=heavy.astype(np.int32),
                groups=groups.astype(np.int32), partial_ofs=partial_ofs.astype(np.int32))


def xsplit(indptr, indices, heavy, n_nodes: int, chunk: int):
    """Source-range split of the heavy rows (plan option xcd_split).

    The node ids split into 8 ranges of R = ceil(N / 8) ids (range r holds
    sources r*R .. (r+1)*R - 1). For each heavy node in the given order, each
    range's part of its (ascending) entries, a contiguous run of len entries
    starting at position a, becomes k = ceil(len / chunk) groups
    (node, a + len*j // k, a + len*(j+1) // k), j = 0..k-1; empty parts give
    none. partial_ofs[k] .. partial_ofs[k+1] are node k's groups. The launch
    order puts the i-th group of range r at slot 8*i + r and -1 in the slots
    a range has no group for, with 8 * (the largest per-range count) slots.

    Returns dict groups int32 [G, 3], partial_ofs int32 [n_heavy + 1],
    order int32 [S]."""
    ip = np.asarray(indptr, np.int64)
    ix = np.asarray(indices, np.int64)
    R = -(-int(n_nodes) // 8)
    span = int(chunk)
    groups, pofs, per_range = [], [0], [[] for _ in range(8)]
    for node in np.asarray(heavy, np.int64):
        e0, e1 = int(ip[node]), int(ip[node + 1])
        src = ix[e0:e1]
        for r in range(8):
            a = e0 + int(np.searchsorted(src, r * R, side="left"))
            b = e1 if r == 7 else e0 + int(np.searchsorted(src, (r + 1) * R, side="left"))
            n = b - a
            if n <= 0:
                continue
            k = -(-n // span)
            for j in range(k):
                per_range[r].append(len(groups))
                groups.append((int(node), a + n * j // k, a + n * (j + 1) // k))
        pofs.append(len(groups))
    most = max(len(l) for l in per_range)
    order = np.full(8 * most, -1, np.int64)
    for r, l in enumerate(per_range):
        order[8 * np.arange(len(l), dtype=np.int64) + r] = l
    g = np.asarray(groups, np.int64).reshape(-1, 3)
    return dict(groups=g.astype(np.int32), partial_ofs=np.asarray(pofs, np.int32), order=order.astype(np.int32))


def launch_order(indptr, light, order: int = 2, threshold: int = 512):
    """Launch order of the light nodes (kernel results do not depend on it).

    order 0: the light list itself; order 1: descending degree; order 2:
    nodes of degree > max(1, threshold // 4) first, by descending
    floor(log2(degree)), then all others; order 3 (the packed launches'
    order): descending ceil(degree / 4); ties by ascending id."""
    ip = np.asarray(indptr, np.int64)
    l = np.asarray(light, np.int64)
    if order == 0:
        return l.astype(np.int32)
    deg = ip[l + 1] - ip[l]
    if order == 1:
        return l[np.lexsort((l, -deg))].astype(np.int32)
    if order == 3:
        steps = (deg + 3) // 4
        return l[np.lexsort((l, -steps))].astype(np.int32)
    hoist = max(1, int(threshold) // 4)
    b = np.floor(np.log2(np.maximum(deg, 1))).astype(np.int64)
    key = np.where(deg > hoist, 63 - b, 64)
    return l[np.lexsort((l, key))].astype(np.int32)


def csc(indptr, indices, n_nodes: int):
    """Transposed adjacency: for each source j, the destinations i of its
    out-edges j -> i in ascending order (with multiplicity).
    Returns (cindptr int32 [N+1], cindices int32 [E])."""
    n = int(n_nodes)
    ip = np.asarray(indptr, np.int64)
    dst = np.repeat(np.arange(n, dtype=np.int64), np.diff(ip))
    src = np.asarray(indices, np.int64)
    keys = np.sort(src * n + dst)
    cols = keys // n
    cindices = (keys - cols * n).astype(np.int32)
    cindptr = np.zeros(n + 1, np.int64)
    np.cumsum(np.bincount(cols, minlength=n), out=cindptr[1:])
    return cindptr.astype(np.int32), cindices


def tile_census(indptr, indices, n_nodes: int, min_nnz: int, threshold: int):
    """16x16 dense-tile census (the pages' block-sparse 16x16 tiles for
    locally dense neighbourhoods).

    Node ids are grouped into aligned blocks of 16. A block pair (destination
    row block b, source column block c) is eligible when no node of row block
    b has in-degree > threshold and no node of column block c has out-degree
    > threshold (heavy rows and sources keep the chunked CSR path). An
    eligible pair holding at least min_nnz distinct (dst, src) positions
    becomes a tile with a 256-bit presence mask: bit (dst % 16) * 16 +
    (src % 16), stored as four uint64 words (word w holds bits 64w..64w+63).
    Tiles are listed by (b, c) ascending. The first occurrence (CSR order) of
    each position inside a tile is represented by the tile; every other edge
    (including repeated copies) stays in the residual CSR, in CSR order.

    Returns dict with
      tile_rc [T,2] int32, tile_mask [T,4] uint64, tile_ptr [NB+1] int32,
      trb: row blocks with tiles, rindptr/rindices: residual CSR,
      light_nt: nodes of in-degree <= threshold in row blocks without tiles,
      ctile [T] int32: tile ids ordered by (c, b), ctile_ptr [NB+1] int32,
      tcb: column blocks with tiles, rcindptr/rcindices: transposed residual,
      c_light_nt: nodes of out-degree <= threshold in column blocks without tiles."""
    n = int(n_nodes)
    nb = (n + 15) // 16
    ip = np.asarray(indptr, np.int64)
    src = np.asarray(indices, np.int64)
    deg = np.diff(ip)
    dst = np.repeat(np.arange(n, dtype=np.int64), deg)
    odeg = np.bincount(src, minlength=n)
    blk = np.arange(n) // 16
    rb_ok = np.bincount(blk, weights=(deg > threshold), minlength=nb) == 0
    cb_ok = np.bincount(blk, weights=(odeg > threshold), minlength=nb) == 0
    pair = (dst // 16) * nb + src // 16
    elig = rb_ok[dst // 16] & cb_ok[src // 16]
    first = np.zeros(src.size, bool)
    if src.size:
        first[np.unique(dst * n + src, return_index=True)[1]] = True
    cand = first & elig
    up, uc = np.unique(pair[cand], return_counts=True)
    tiles = up[uc >= min_nnz]
    in_tile = cand & np.isin(pair, tiles)
    mask = np.zeros((tiles.size, 4), np.uint64)
    if tiles.size:
        t = np.searchsorted(tiles, pair[in_tile])
        bit = (dst[in_tile] % 16) * 16 + (src[in_tile] % 16)
        val = np.left_shift(np.uint64(1), (bit % 64).astype(np.uint64))
        np.bitwise_or.at(mask, (t, bit // 64), val)
    trow, tcol = tiles // nb, tiles % nb
    tile_ptr = np.zeros(nb + 1, np.int64)
    np.cumsum(np.bincount(trow, minlength=nb), out=tile_ptr[1:])
    keep = ~in_tile
    rindptr = np.zeros(n + 1, np.int64)
    np.cumsum(np.bincount(dst[keep], minlength=n), out=rindptr[1:])
    rindices = src[keep]
    rb_has = np.diff(tile_ptr) > 0
    light_nt = np.nonzero((deg <= threshold) & ~rb_has[blk])[0]
    ctile = np.lexsort((trow, tcol)) if tiles.size else np.zeros(0, np.int64)
    ctile_ptr = np.zeros(nb + 1, np.int64)
    np.cumsum(np.bincount(tcol, minlength=nb), out=ctile_ptr[1:])
    cb_has = np.diff(ctile_ptr) > 0
    rcindptr, rcindices = csc(rindptr, rindices, n)
    c_light_nt = np.nonzero((odeg <= threshold) & ~cb_has[blk])[0]
    i32 = lambda a: np.asarray(a).astype(np.int32)
    return dict(tile_rc=i32(np.stack([trow, tcol], axis=1).reshape(-1, 2)), tile_mask=mask,
                tile_ptr=i32(tile_ptr), trb=i32(np.nonzero(rb_has)[0]), rindptr=i32(rindptr),
                rindices=i32(rindices), light_nt=i32(light_nt), ctile=i32(ctile), ctile_ptr=i32(ctile_ptr),
                tcb=i32(np.nonzero(cb_has)[0]), rcindptr=rcindptr, rcindices=rcindices,
                c_light_nt=i32(c_light_nt))


# ---------------------------------------------------------------------------
# floating point (fp64)
# ---------------------------------------------------------------------------

def _rows(rows, n):
    if rows is None:
        return None, n
    r = np.ascontiguousarray(rows, np.int64)
    if r.size and (r.min() < 0 or r.max() >= n):
        raise ValueError("row out of range")
    return r, r.size


def _graph(indptr, indices):
    return np.ascontiguousarray(indptr, np.int64), np.ascontiguousarray(indices, np.int32)


def gt_fwd(indptr, indices, Q, K, V, scale: Optional[float] = None, rows=None):
    """Graph-Transformer forward in fp64.

    s_ij = scale * <q_i, k_j> per head (scale = 1/sqrt(D) by default);
    alpha_ij = softmax over j in N(i); O_i = sum_j alpha_ij v_j;
    LSE_i = m_i + ln sum_j exp(s_ij - m_i).
    Returns dict O [r,H,D], LSE [r,H], SO [r,H,D], SL [r,H] (scales)."""
    Q, K, V = _f64(Q), _f64(K), _f64(V)
    N, H, D = Q.shape
    ip, ix = _graph(indptr, indices)
    sc = 1.0 / np.sqrt(D) if scale is None else float(scale)
    r, nr = _rows(rows, N)
    O = np.empty((nr, H, D)); LSE = np.empty((nr, H)); SO = np.empty((nr, H, D)); SL = np.empty((nr, H))
    rc = _load().orc_gt_fwd(N, _p(ip), _p(ix), H, D, _p(Q), _p(K), _p(V), sc, nr, _p(r),
                            _p(O), _p(LSE), _p(SO), _p(SL))
    if rc:
        raise MemoryError("oracle row buffer")
    return dict(O=O, LSE=LSE, SO=SO, SL=SL)


def gatv2_fwd(indptr, indices, XD, XS, att, V=None, slope: float = 0.2, rows=None):
    """GATv2 forward in fp64.

    s_ij = sum_d a[h,d] * LeakyReLU_slope(xs_j + xd_i) per head (no scale);
    the same softmax; O_i = sum_j alpha_ij v_j with v = xs unless V is given."""
    XD, XS = _f64(XD), _f64(XS)
    Vv = XS if V is None else _f64(V)
    a = _f64(att)
    N, H, D = XD.shape
    ip, ix = _graph(indptr, indices)
    r, nr = _rows(rows, N)
    O = np.empty((nr, H, D)); LSE = np.empty((nr, H)); SO = np.empty((nr, H, D)); SL = np.empty((nr, H))
    rc = _load().orc_gatv2_fwd(N, _p(ip), _p(ix), H, D, _p(XD), _p(XS), _p(Vv), _p(a), float(slope),
                               nr, _p(r), _p(O), _p(LSE), _p(SO), _p(SL))
    if rc:
        raise MemoryError("oracle row buffer")
    return dict(O=O, LSE=LSE, SO=SO, SL=SL)


def gt_bwd_dst(indptr, indices, Q, K, V, dO, scale: Optional[float] = None, rows=None):
    """Destination side of the Graph-Transformer backward in fp64, from the
    definition, for the rows `rows` (None = all): dQ, Delta (from the
    weights), the scale SdQ, and the row statistics M (max logit) and Z (sum
    of exp(s - M)) that the source side needs. Returns a dict of those."""
    Q, K, V, dO = _f64(Q), _f64(K), _f64(V), _f64(dO)
    N, H, D = Q.shape
    ip, ix = _graph(indptr, indices)
    sc = 1.0 / np.sqrt(D) if scale is None else float(scale)
    r, nr = _rows(rows, N)
    dQ = np.empty((nr, H, D)); Dl = np.empty((nr, H)); M = np.empty((nr, H)); Z = np.empty((nr, H))
    SdQ = np.empty((nr, H, D))
    rc = _load().orc_gt_bwd_rows(N, _p(ip), _p(ix), H, D, _p(Q), _p(K), _p(V), _p(dO), sc, nr, _p(r),
                                 _p(dQ), _p(Dl), _p(M), _p(Z), _p(SdQ))
    if rc:
        raise MemoryError("oracle row buffer")
    return dict(dQ=dQ, Delta=Dl, SdQ=SdQ, M=M, Z=Z)


def gt_bwd_src(cindptr, cindices, Q, K, V, dO, M, Z, Delta, scale: Optional[float] = None, srcs=None,
               need=None):
    """Source side of the Graph-Transformer backward in fp64 over the
    transposed adjacency (cindptr/cindices list each source's destinations):
    dK, dV and their scales SdK, SdV for the sources `srcs` (None = all).
    M, Z, Delta are the destination statistics of gt_bwd_dst, for every row
    (need None) or for the rows listed in `need` (in that order)."""
    Q, K, V, dO = _f64(Q), _f64(K), _f64(V), _f64(dO)
    N, H, D = Q.shape
    sc = 1.0 / np.sqrt(D) if scale is None else float(scale)
    cip = np.ascontiguousarray(cindptr, np.int64)
    cix = np.ascontiguousarray(cindices, np.int32)
    s, ns = _rows(srcs, N)
    if need is None:
        slot = np.arange(N, dtype=np.int64)
    else:
        slot = np.full(N, -1, np.int64)
        slot[np.asarray(need, np.int64)] = np.arange(len(need))
    M, Z, Dl = (np.ascontiguousarray(a, np.float64) for a in (M, Z, Delta))
    dK = np.empty((ns, H, D)); dV = np.empty((ns, H, D)); SdK = np.empty((ns, H, D)); SdV = np.empty((ns, H, D))
    rc = _load().orc_gt_bwd_srcs(N, _p(cip), _p(cix), H, D, _p(Q), _p(K), _p(V), _p(dO), sc, _p(slot),
                                 _p(M), _p(Z), _p(Dl), ns, _p(s), _p(dK), _p(dV), _p(SdK), _p(SdV))
    if rc:
        raise RuntimeError("oracle source pass: missing destination statistics")
    return dict(dK=dK, dV=dV, SdK=SdK, SdV=SdV)


def gt_bwd(indptr, indices, Q, K, V, dO, scale: Optional[float] = None, rows=None, srcs=None,
           csc_arrays=None, want_src: bool = True):
    """Graph-Transformer backward in fp64, from the definition.

    dQ (and Delta) for the destination rows `rows` (None = all); dK, dV for
    the sources `srcs` (None = all) over the transposed adjacency. The
    destination statistics the source side needs are computed for exactly the
    rows it touches. Returns dict dQ, Delta, SdQ [rows] and dK, dV, SdK, SdV
    [srcs]."""
    Q, K, V, dO = _f64(Q), _f64(K), _f64(V), _f64(dO)
    N = Q.shape[0]
    ip, ix = _graph(indptr, indices)
    d = gt_bwd_dst(ip, ix, Q, K, V, dO, scale, rows)
    out = dict(dQ=d["dQ"], Delta=d["Delta"], SdQ=d["SdQ"])
    if not want_src:
        return out
    cip, cix = csc(ip, ix, N) if csc_arrays is None else csc_arrays
    cip = np.ascontiguousarray(cip, np.int64)
    cix = np.ascontiguousarray(cix, np.int32)
    s, _ = _rows(srcs, N)
    if rows is None:
        stats, need = d, None
    else:
        # destination rows touched by the listed sources
        if s is None:
            need = np.arange(N, dtype=np.int64)
        else:
            parts = [cix[cip[j]:cip[j + 1]] for j in s]
            need = np.unique(np.concatenate(parts).astype(np.int64)) if parts else np.zeros(0, np.int64)
        stats = gt_bwd_dst(ip, ix, Q, K, V, dO, scale, need)
    out.update(gt_bwd_src(cip, cix, Q, K, V, dO, stats["M"], stats["Z"], stats["Delta"], scale, s, need))
    return out


def gatv2_bwd(indptr, indices, XD, XS, att, dO, V=None, slope: float = 0.2, rows=None, srcs=None,
              csc_arrays=None, want_src: bool = True, want_da: bool = True):
    """GATv2 backward in fp64, from the definition.

    Returns dict with dXD, Delta, SdXD for `rows` (None = all); dXS (score
    path plus, when V is XS, the value path), dV (value path, only when V is
    separate) and their scales for `srcs`; and, with want_da, d_att [H, D]
    summed over every edge of the graph (with its scale)."""
    XD, XS, dO, a = _f64(XD), _f64(XS), _f64(dO), _f64(att)
    alias = V is None
    Vv = XS if alias else _f64(V)
    N, H, D = XD.shape
    ip, ix = _graph(indptr, indices)
    lib = _load()

    def rows_pass(r, nr):
        out = [np.empty((nr, H, D)), np.empty((nr, H)), np.empty((nr, H)), np.empty((nr, H)),
               np.empty((nr, H, D)), np.empty((nr, H, D)), np.empty((nr, H, D))]
        rc = lib.orc_gatv2_bwd_rows(N, _p(ip), _p(ix), H, D, _p(XD), _p(XS), _p(Vv), _p(a), float(slope), _p(dO),
                                    nr, _p(r), *[_p(o) for o in out])
        if rc:
            raise MemoryError("oracle row buffer")
        return out

    r, nr = _rows(rows, N)
    dXD, Dl, M, Z, DA, SdXD, SDA = rows_pass(r, nr)
    res = dict(dXD=dXD, Delta=Dl, SdXD=SdXD)
    if want_da:
        if r is None:
            DAall, SDAall = DA, SDA
        else:
            _, _, _, _, DAall, _, SDAall = rows_pass(None, N)
        res["d_att"] = DAall.sum(axis=0)
        res["Sd_att"] = SDAall.sum(axis=0)
    if not want_src:
        return res
    cip, cix = csc(ip, ix, N) if csc_arrays is None else csc_arrays
    cip = np.ascontiguousarray(cip, np.int64)
    cix = np.ascontiguousarray(cix, np.int32)
    s, ns = _rows(srcs, N)
    if s is None:
        need = np.arange(N, dtype=np.int64)
    else:
        parts = [cix[cip[j]:cip[j + 1]] for j in s]
        need = np.unique(np.concatenate(parts).astype(np.int64)) if parts else np.zeros(0, np.int64)
    if r is None and s is None:
        M2, Z2, D2 = M, Z, Dl
    else:
        _, D2, M2, Z2, _, _, _ = rows_pass(need, need.size)
    slot = np.full(N, -1, np.int64)
    slot[need] = np.arange(need.size)
    dXS = np.empty((ns, H, D)); dV = np.empty((ns, H, D)); SdXS = np.empty((ns, H, D)); SdV = np.empty((ns, H, D))
    rc = lib.orc_gatv2_bwd_srcs(N, _p(cip), _p(cix), H, D, _p(XD), _p(XS), _p(Vv), _p(a), float(slope), _p(dO),
                                _p(slot), _p(M2), _p(Z2), _p(D2), ns, _p(s), _p(dXS), _p(dV), _p(SdXS), _p(SdV))
    if rc:
        raise RuntimeError("oracle source pass: missing destination statistics")
    if alias:
        res.update(dXS=dXS + dV, SdXS=SdXS + SdV)
    else:
        res.update(dXS=dXS, SdXS=SdXS, dV=dV, SdV=SdV)
    return res


# ---------------------------------------------------------------------------
# cached SpMM aggregation (GCN / GraphConv)
# ---------------------------------------------------------------------------
SPMM_NORMS = {"sum": 0, "mean": 1, "gcn": 2}


def spmm_weights(indptr, indices, norm: str = "gcn") -> np.ndarray:
    """Per-entry weights w_e of entry e = (row i, source j), CSR order, fp64:
    "sum" 1; "mean" 1 / indeg(i); "gcn" d(i) d(j) with d(v) = indeg(v)^-1/2,
    taken as 0 for a node without entries (a source whose own row is empty
    contributes nothing), indeg the number of row entries (self-loops
    included when the CSR holds them, i.e. the degrees of A + I)."""
    ip = np.asarray(indptr, np.int64)
    ix = np.asarray(indices, np.int64)
    deg = np.diff(ip).astype(np.float64)
    rows = np.repeat(np.arange(ip.size - 1), np.diff(ip))
    if norm == "sum":
        return np.ones(ix.size)
    if norm == "mean":
        return 1.0 / deg[rows]
    if norm == "gcn":
        dinv = np.zeros_like(deg)
        dinv[deg > 0] = 1.0 / np.sqrt(deg[deg > 0])
        return dinv[rows] * dinv[ix]
    raise ValueError(norm)


def spmm(indptr, indices, X, norm: str = "gcn", transpose: bool = False, rows=None):
    """Y = A_w X (or A_w^T X) in fp64 with the weights of spmm_weights, A_w
    the N x N sparse matrix with entry (i, j) += w_e per CSR entry (repeats
    add up). scipy's sparse product is the reduction. Returns dict Y [N, F]
    (or only the listed rows) and the summation scale S = |A_w| |X|."""
    import scipy.sparse as sp
    ip = np.asarray(indptr, np.int64)
    ix = np.asarray(indices, np.int64)
    n = ip.size - 1
    X = np.asarray(X, np.float64).reshape(n, -1)
    A = sp.csr_matrix((spmm_weights(ip, ix, norm), ix, ip), shape=(n, n))
    if transpose:
        A = A.T.tocsr()
    if rows is not None:
        A = A[np.asarray(rows, np.int64)]
    return dict(Y=A @ X, S=abs(A) @ np.abs(X))


# ---------------------------------------------------------------------------
# graph reordering
# ---------------------------------------------------------------------------
ORDERS = {"degree": 0, "rcm": 1}


def total_degree(indptr, indices, n_nodes: int) -> np.ndarray:
    """deg(v) = entries of v's row (in-degree) + entries naming v (out-degree)."""
    ip = np.asarray(indptr, np.int64)
    return np.diff(ip) + np.bincount(np.asarray(indices, np.int64), minlength=n_nodes)[:n_nodes]


def reorder(indptr, indices, n_nodes: int, method: str = "rcm") -> np.ndarray:
    """Node order for relabelling, as perm[new id] = old id (int32).

    "degree": descending total degree, ties by ascending id.
    "rcm": reverse Cuthill-McKee on the symmetrised graph (a node's
    neighbours are its row's sources and the rows naming it). Cuthill-McKee
    visits components one after another, each from its unvisited node of
    smallest (degree, id), breadth first: when a node is taken from the
    queue its not yet visited neighbours are appended in ascending (degree,
    id). The permutation is that visiting order reversed. Plain queue code
    (pure Python loops: small and medium graphs only)."""
    n = int(n_nodes)
    ip = np.asarray(indptr, np.int64)
    ix = np.asarray(indices, np.int64)
    deg = total_degree(ip, ix, n)
    if method == "degree":
        return np.lexsort((np.arange(n), -deg)).astype(np.int32)
    if method != "rcm":
        raise ValueError(method)
    # symmetrised adjacency: in-neighbours (row) and out-neighbours (column)
    rows = np.repeat(np.arange(n, dtype=np.int64), np.diff(ip))
    src = np.concatenate([ix, rows])
    dst = np.concatenate([rows, ix])
    o = np.argsort(dst, kind="stable")
    nb = src[o]
    nptr = np.concatenate([[0], np.cumsum(np.bincount(dst, minlength=n))])
    key = deg * n + np.arange(n)                       # (degree, id) as one sortable number
    visited = np.zeros(n, bool)
    order = []
    starts = np.argsort(key, kind="stable")            # candidate start nodes by (degree, id)
    si = 0
    from collections import deque
    while len(order) < n:
        while visited[starts[si]]:
            si += 1
        s = int(starts[si])
        visited[s] = True
        order.append(s)
        q = deque([s])
        while q:
            u = q.popleft()
            cand = np.unique(nb[nptr[u]:nptr[u + 1]])
            cand = cand[~visited[cand]]
            cand = cand[np.argsort(key[cand], kind="stable")]
            for v in cand:
                visited[v] = True
                order.append(int(v))
                q.append(int(v))
    return np.asarray(order[::-1], np.int32)


def permute_graph(indptr, indices, perm):
    """CSR of the relabelled graph: new row r is old row perm[r], each source
    j renamed to its new id, rows sorted ascending (entries kept, repeats
    included). Returns (indptr int32, indices int32)."""
    perm = np.asarray(perm, np.int64)
    n = perm.size
    inv = np.empty(n, np.int64)
    inv[perm] = np.arange(n)
    ip = np.asarray(indptr, np.int64)
    ix = np.asarray(indices, np.int64)
    rows_old = np.repeat(np.arange(n, dtype=np.int64), np.diff(ip))
    r = inv[rows_old]
    c = inv[ix]
    o = np.lexsort((c, r))
    new_ip = np.concatenate([[0], np.cumsum(np.bincount(r, minlength=n))]).astype(np.int32)
    return new_ip, c[o].astype(np.int32)


def bandwidth(indptr, indices) -> int:
    """max |i - j| over the entries (i, j) of the CSR (0 for no entries)."""
    ip = np.asarray(indptr, np.int64)
    ix = np.asarray(indices, np.int64)
    if ix.size == 0:
        return 0
    rows = np.repeat(np.arange(ip.size - 1), np.diff(ip))
    return int(np.max(np.abs(rows - ix)))


# ---------------------------------------------------------------------------
# degree-aware reduction layer
# ---------------------------------------------------------------------------
REDUCE_OPS = {"max": 0, "min": 1}
REDUCE_MSGS = {"src": 0, "diff": 1}


def segment_reduce(indptr, indices, X, op: str = "max", msg: str = "src", rows=None):
    """Neighbourhood max / min of per-edge messages with the winning source.

    m_ij = X[j] (msg "src") or X[j] - X[i] (msg "diff", one fp32
    subtraction); out[i, f] = max (or min) over row i's entries of m_ij[f];
    arg[i, f] = the smallest j attaining it (-0 == +0); empty rows give 0 and
    -1. X is [N, F] (or [N, H, D], flattened per node) fp32 values, bf16
    inputs widened. Decided in fp32, the precision of the messages.
    Returns dict out float32 [r, F], arg int32 [r, F]."""
    X = np.ascontiguousarray(X, np.float32)
    N = X.shape[0]
    X = X.reshape(N, -1)
    F = X.shape[1]
    ip, ix = _graph(indptr, indices)
    r, nr = _rows(rows, N)
    out = np.empty((nr, F), np.float32)
    arg = np.empty((nr, F), np.int32)
    rc = _load().orc_segment_reduce(N, _p(ip), _p(ix), F, _p(X), REDUCE_OPS[op], REDUCE_MSGS[msg], nr, _p(r),
                                    _p(out), _p(arg))
    if rc:
        raise MemoryError("oracle row buffer")
    return dict(out=out, arg=arg)


def segment_reduce_bwd(indptr, indices, dOut, arg, msg: str = "src", n_nodes: Optional[int] = None,
                       want_scale: bool = False, rows=None):
    """Gradient of segment_reduce in fp64: each (i, f) with a winner j sends
    dOut[i, f] to X[j, f], and for msg "diff" also -dOut[i, f] to X[i, f]
    (the message is X[j] - X[i]). A source that appears several times in a
    row receives the gradient once, through the winning entry.
    dOut and arg hold rows 0..N-1, or the rows listed in `rows` (then only
    their terms are summed). Returns dX float64 [N, F]; with want_scale also
    the summation scale S = the sum of |terms| added into each element."""
    dOut = np.asarray(dOut, np.float64)
    arg = np.asarray(arg, np.int64)
    N = int(n_nodes if n_nodes is not None else dOut.shape[0])
    dOut = dOut.reshape(dOut.shape[0], -1)
    arg = arg.reshape(arg.shape[0], -1)
    F = dOut.shape[1]
    dX = np.zeros((N, F), np.float64)
    won = arg >= 0
    r_idx, f_idx = np.nonzero(won)
    i_idx = r_idx if rows is None else np.asarray(rows, np.int64)[r_idx]
    np.add.at(dX, (arg[r_idx, f_idx], f_idx), dOut[r_idx, f_idx])
    if msg == "diff":
        np.add.at(dX, (i_idx, f_idx), -dOut[r_idx, f_idx])
    if not want_scale:
        return dX
    S = np.zeros((N, F), np.float64)
    np.add.at(S, (arg[r_idx, f_idx], f_idx), np.abs(dOut[r_idx, f_idx]))
    if msg == "diff":
        np.add.at(S, (i_idx, f_idx), np.abs(dOut[r_idx, f_idx]))
    return dX, S


def round_bf16(x) -> np.ndarray:
    """fp32 values rounded to the nearest bf16 (ties to even), returned as
    fp32 (finite inputs)."""
    b = np.ascontiguousarray(x, np.float32).view(np.uint32).astype(np.uint64)
    b = (b + 0x7FFF + ((b >> 16) & 1)) >> 16
    return (b.astype(np.uint32) << 16).view(np.float32)


def normwise_error(x, ref) -> float:
    """Plain normwise relative error max_e |x_e - r_e| / max_e |r_e| over
    the finite entries of ref (reported beside the scaled error; 0 when ref
    has no non-zero finite entry and x equals it there)."""
    x = np.asarray(x, np.float64)
    ref = np.asarray(ref, np.float64)
    fin = np.isfinite(ref)
    if not np.any(fin):
        return 0.0
    num = float(np.max(np.abs(x[fin] - ref[fin])))
    den = float(np.max(np.abs(ref[fin])))
    return num / den if den > 0 else (0.0 if num == 0 else float("inf"))


def scaled_error(x, ref, scale) -> float:
    """max_e |x_e - r_e| / max(|r_e|, S_e), S_e the oracle's summation scale
    (where both |r_e| and S_e are 0 the absolute difference is taken).

    Entries where both are infinite with the same sign (empty rows' LSE)
    count as exact; an infinity on one side only, infinities of opposite
    signs and NaN on either side give an infinite error."""
    x = np.asarray(x, np.float64)
    ref = np.asarray(ref, np.float64)
    if ref.size == 0:
        return 0.0
    s = np.maximum(np.abs(ref), np.asarray(scale, np.float64))
    same_inf = np.isinf(x) & np.isinf(ref) & (np.sign(x) == np.sign(ref))
    bad = ~same_inf & ~(np.isfinite(x) & np.isfinite(ref) & np.isfinite(s))
    ok = ~(same_inf | bad)
    diff = np.where(ok, np.abs(np.where(ok, x, 0.0) - np.where(ok, ref, 0.0)), 0.0)
    den = np.where(ok & (s > 0), s, 1.0)
    e = np.where(bad, np.inf, diff / den)
    return float(np.max(e))
