"""Seeded synthetic workloads for fused CSR neighbourhood attention.

This module draws graphs (as COO edge lists) and node features. It holds none
of the attention method's arithmetic: no CSR construction, no scores, no
softmax. Both the fp64 oracle (``oracle/``) and the HIP library
(``io_aware_sparse_amd``) consume what it produces; neither is imported here.

The pages evaluate on OGB graphs, citation networks and GraphLand industrial
graphs ("On Efficient Scaling of GNNs via IO-Aware Layers Implementations",
technical summary, Results). None of those datasets is available, so each
workload below is a seeded stand-in with the shape, size and degree structure
of the case it names:

  gt_uniform_n2708        uniform random digraph, 10,556 distinct pairs
                          (citation-graph sized), H=1, D=16, fp32
  gt_chunglu25_n169k      Chung-Lu, degree exponent 2.5, w_max 13,000,
                          1.17M pairs, H=4, D=32, fp32
  gatv2_zipf21_n100k      in-degrees round(s*Zipf(2.1)) capped at 50,000,
                          mean 50, H=8, D=16, fp32, a ~ N(0, 1/D)
  gt_chunglu22_n2450k     Chung-Lu, degree exponent 2.2, w_max 20,000,
                          62M pairs, H=4, D=32, bf16
  gt_comm16_n1m_deg100    16-node dense communities + 84 random
                          inter-community in-edges per node, H=8, D=64, bf16,
                          with an upstream gradient
  gt_comm16_n1m_deg27     same communities + 11 inter-community in-edges
  maxpool_zipf21_n100k    the Zipf(2.1) graph with F = 128 fp32 features per
                          node, for the neighbourhood max / min reduction
  maxpool_chunglu22_n2450k  the degree-2.2 Chung-Lu graph with F = 128 bf16
  spmm_chunglu25_n169k    the degree-2.5 Chung-Lu graph, F = 128 fp32, for
                          the SpMM aggregation (GCN / GraphConv)
  spmm_chunglu22_n2450k   the degree-2.2 Chung-Lu graph, F = 128 bf16
  spmm_comm16_n1m_deg27   the clustered graph with 11 inter-community sources,
                          F = 128 bf16 (the graph the 16x16 block path targets)

Self-loops are never emitted here; the CSR builder adds exactly one per node.

Every bulk draw is split into fixed chunks of ``_CHUNK`` values, each with its
own spawned seed, and filled on a thread pool: the result depends only on the
seed, never on the thread count.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field
from typing import Dict, Optional

import numpy as np

_CHUNK = 1 << 22


def _threads() -> int:
    n = os.environ.get("OMP_NUM_THREADS")
    try:
        k = int(n) if n else (os.cpu_count() or 1)
    except ValueError:
        k = os.cpu_count() or 1
    return max(1, min(k, 16))


def _chunked(ss: np.random.SeedSequence, n: int, fill):
    """Run ``fill(rng, out_slice)`` over fixed chunks of an n-element draw."""
    nch = max(1, (n + _CHUNK - 1) // _CHUNK)
    kids = ss.spawn(nch)

    def job(k):
        lo = k * _CHUNK
        hi = min(n, lo + _CHUNK)
        return fill(np.random.default_rng(kids[k]), lo, hi)

    if nch == 1:
        job(0)
        return
    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(job, range(nch)))


def normal_f32(ss: np.random.SeedSequence, shape, std: float = 1.0,
               bf16: bool = False):
    """N(0, std^2) fp32 draws of the given shape.

    With bf16=True the values are rounded to bf16 (round-to-nearest-even)
    chunk by chunk, and (bits uint16, values fp32) is returned."""
    n = int(np.prod(shape))
    out = np.empty(n, np.float32)
    bits = np.empty(n, np.uint16) if bf16 else None

    def fill(rng, lo, hi):
        o = out[lo:hi]
        rng.standard_normal(hi - lo, dtype=np.float32, out=o)
        if std != 1.0:
            o *= np.float32(std)
        if bf16:
            bits[lo:hi], o[:] = round_to_bf16(o)

    _chunked(ss, n, fill)
    if bf16:
        return bits.reshape(shape), out.reshape(shape)
    return out.reshape(shape)


def _sample_weighted(ss: np.random.SeedSequence, cdf: np.ndarray, n: int) -> np.ndarray:
    """n iid draws of an index with P(i) proportional to the weights behind cdf."""
    out = np.empty(n, np.int64)

    def fill(rng, lo, hi):
        u = rng.random(hi - lo)
        out[lo:hi] = np.searchsorted(cdf, u, side="right")

    _chunked(ss, n, fill)
    np.minimum(out, cdf.size - 1, out=out)
    return out


def _uniform_int(ss: np.random.SeedSequence, high: np.ndarray | int, n: int) -> np.ndarray:
    """n draws uniform in [0, high) (high may be per-draw)."""
    out = np.empty(n, np.int64)
    hi_arr = np.broadcast_to(np.asarray(high, np.int64), (n,))

    def fill(rng, lo, hi):
        out[lo:hi] = rng.integers(0, hi_arr[lo:hi])

    _chunked(ss, n, fill)
    return out


def round_to_bf16(x: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Round fp32 values to bf16 (round-to-nearest-even).

    Returns (bits as uint16, the same values widened back to fp32). Inputs are
    finite normal-range draws, so no NaN handling is needed."""
    b = np.ascontiguousarray(x, np.float32).view(np.uint32)
    t = b >> 16
    t &= 1
    t += 0x7FFF
    t += b
    t >>= 16
    hi = t.astype(np.uint16)
    t <<= 16
    return hi, t.view(np.float32)


@dataclass
class Workload:
    name: str
    kind: str                 # "gt" (dot-product), "gatv2", "reduce" (max / min of X) or "spmm" (A_w X)
    n_nodes: int
    src: np.ndarray           # int32 [E0], edge src -> dst, no self-pairs
    dst: np.ndarray           # int32 [E0]
    heads: int
    dim: int
    dtype: str                # "f32" or "bf16"
    backward: bool            # workload includes the gradient pass
    feats: Dict[str, np.ndarray] = field(default_factory=dict)   # fp32 [N,H,D], dtype-rounded
    bits: Dict[str, np.ndarray] = field(default_factory=dict)    # uint16 bf16 bits, bf16 only
    att: Optional[np.ndarray] = None                             # [H,D] fp32 (GATv2)
    seed: int = 0
    meta: Dict[str, float] = field(default_factory=dict)

    @property
    def n_edges_in(self) -> int:
        return int(self.src.size)


# --------------------------------------------------------------------------
# graph generators
# --------------------------------------------------------------------------

def chung_lu_weights(n: int, gamma: float, w_max: float, w_sum: float) -> np.ndarray:
    """w_i = c * (i + i0)^(-1/(gamma-1)) with w_0 = w_max and sum w = w_sum.

    i0 is found by bisection (the sum falls monotonically as i0 grows once c is
    tied to w_max), then c = w_max * i0^beta."""
    beta = 1.0 / (gamma - 1.0)
    i = np.arange(n, dtype=np.float64)

    def total(i0):
        return w_max * np.sum(((i + i0) / i0) ** (-beta))

    lo, hi = 1e-6, 1e7
    for _ in range(200):
        mid = np.sqrt(lo * hi)
        if total(mid) > w_sum:
            hi = mid
        else:
            lo = mid
    i0 = np.sqrt(lo * hi)
    return w_max * ((i + i0) / i0) ** (-beta)


def _merge_unique(keys: np.ndarray, new: np.ndarray) -> np.ndarray:
    """Sorted union of a sorted unique array and a batch of new keys."""
    new = np.unique(new)
    if keys.size == 0:
        return new
    pos = np.searchsorted(keys, new)
    hit = (pos < keys.size) & (keys[np.minimum(pos, keys.size - 1)] == new)
    return np.insert(keys, pos[~hit], new[~hit])


def _chung_lu_pairs(ss, n, gamma, w_max, n_pairs):
    w = chung_lu_weights(n, gamma, w_max, float(n_pairs))
    cdf = np.cumsum(w)
    cdf /= cdf[-1]
    kids = ss.spawn(64)
    keys = np.empty(0, np.int64)
    k = 0
    while keys.size < n_pairs:
        draw = n_pairs if k == 0 else int((n_pairs - keys.size) * 1.1) + 1024
        s = _sample_weighted(kids[2 * k], cdf, draw)
        d = _sample_weighted(kids[2 * k + 1], cdf, draw)
        keep = s != d
        keys = _merge_unique(keys, d[keep] * n + s[keep])
        k += 1
        if 2 * k + 1 >= len(kids) - 1:
            raise RuntimeError("Chung-Lu top-up did not converge")
    if keys.size > n_pairs:
        rng = np.random.default_rng(kids[-1])
        drop = rng.choice(keys.size, keys.size - n_pairs, replace=False)
        keys = np.delete(keys, drop)
    return (keys % n).astype(np.int64), (keys // n).astype(np.int64), w


def _distinct_sources(ss, n, deg, forbid_lo, forbid_len):
    """For each node i, deg[i] distinct sources uniform over [0, n) minus the
    forbidden block [forbid_lo[i], forbid_lo[i] + forbid_len[i]).

    Rows are drawn in bulk and redrawn where duplicates appear; rows asking for
    more than a tenth of the allowed range use a per-row draw without
    replacement instead."""
    deg = np.asarray(deg, np.int64)
    n_ok = n - np.asarray(forbid_len, np.int64)
    flo = np.asarray(forbid_lo, np.int64)
    flen = np.asarray(forbid_len, np.int64)
    if np.any(deg > n_ok):
        raise ValueError("degree exceeds the number of allowed sources")
    big = deg * 10 > n_ok
    kids = ss.spawn(3)
    rows_src = []
    rows_dst = []
    # per-row draws for the few huge rows
    rng_big = np.random.default_rng(kids[0])
    for i in np.nonzero(big)[0]:
        v = rng_big.choice(n_ok[i], deg[i], replace=False).astype(np.int64)
        v = v + flen[i] * (v >= flo[i])
        rows_src.append(v)
        rows_dst.append(np.full(deg[i], i, np.int64))
    small = np.nonzero(~big & (deg > 0))[0]
    rounds = kids[1].spawn(256)
    pending = small                      # rows still short of their degree
    have = np.empty(0, np.int64)         # distinct keys row*n+src of pending rows
    done = []
    r = 0
    while pending.size:
        cnt = np.bincount(have // n, minlength=n)[pending] if have.size else np.zeros(pending.size, np.int64)
        need = deg[pending] - cnt
        rid = np.repeat(pending, need)
        v = _uniform_int(rounds[r], n_ok[rid], rid.size)
        v = v + flen[rid] * (v >= flo[rid])
        have = _merge_unique(have, rid * n + v)
        cnt = np.bincount(have // n, minlength=n)
        full = cnt[have // n] == deg[have // n]
        done.append(have[full])
        have = have[~full]
        pending = np.unique(have // n) if have.size else have
        r += 1
        if r >= len(rounds):
            raise RuntimeError("distinct-source draw did not converge")
    keys = np.concatenate(done) if done else np.empty(0, np.int64)
    rows_src.append(keys % n)
    rows_dst.append(keys // n)
    return np.concatenate(rows_src), np.concatenate(rows_dst)


def zipf_in_degrees(ss, n, exponent, mean, cap):
    """d_i = min(cap, max(1, round(s * z_i))), z_i ~ Zipf(exponent), with the
    scale s bisected so that the realised mean of d is as close to `mean` as
    the rounding allows."""
    rng = np.random.default_rng(ss)
    z = rng.zipf(exponent, n).astype(np.float64)

    def deg(s):
        return np.minimum(cap, np.maximum(1, np.rint(s * z))).astype(np.int64)

    lo, hi = 1e-3, 1e6
    for _ in range(200):
        mid = 0.5 * (lo + hi)
        if deg(mid).mean() < mean:
            lo = mid
        else:
            hi = mid
    d_lo, d_hi = deg(lo), deg(hi)
    s = hi if abs(d_hi.mean() - mean) <= abs(d_lo.mean() - mean) else lo
    return deg(s), s


def _relabel(ss, n, src, dst):
    perm = np.random.default_rng(ss).permutation(n).astype(np.int64)
    return perm[src], perm[dst]


# --------------------------------------------------------------------------
# workloads
# --------------------------------------------------------------------------

SPECS = {
    "gt_uniform_n2708": dict(seed=1001, kind="gt", n=2708, heads=1, dim=16, dtype="f32", backward=False),
    "gt_chunglu25_n169k": dict(seed=1002, kind="gt", n=169_343, heads=4, dim=32, dtype="f32", backward=False),
    "gatv2_zipf21_n100k": dict(seed=1003, kind="gatv2", n=100_000, heads=8, dim=16, dtype="f32", backward=False),
    "gt_chunglu22_n2450k": dict(seed=1004, kind="gt", n=2_450_000, heads=4, dim=32, dtype="bf16", backward=False),
    "gt_comm16_n1m_deg100": dict(seed=1005, kind="gt", n=1_000_000, heads=8, dim=64, dtype="bf16", backward=True),
    "gt_comm16_n1m_deg27": dict(seed=1005, kind="gt", n=1_000_000, heads=8, dim=64, dtype="bf16", backward=True),
    # neighbourhood max / min reduction on the graphs above (same recipe and seed, hence the same graph)
    "maxpool_zipf21_n100k": dict(seed=1003, kind="reduce", graph="gatv2_zipf21_n100k", n=100_000, heads=1,
                                 dim=128, dtype="f32", backward=False),
    "maxpool_chunglu22_n2450k": dict(seed=1004, kind="reduce", graph="gt_chunglu22_n2450k", n=2_450_000,
                                     heads=1, dim=128, dtype="bf16", backward=False),
    # SpMM aggregation (GCN / GraphConv) on the Chung-Lu graphs
    "spmm_chunglu25_n169k": dict(seed=1002, kind="spmm", graph="gt_chunglu25_n169k", n=169_343, heads=1,
                                 dim=128, dtype="f32", backward=False),
    "spmm_chunglu22_n2450k": dict(seed=1004, kind="spmm", graph="gt_chunglu22_n2450k", n=2_450_000, heads=1,
                                  dim=128, dtype="bf16", backward=False),
    "spmm_comm16_n1m_deg27": dict(seed=1005, kind="spmm", graph="gt_comm16_n1m_deg27", n=1_000_000, heads=1,
                                  dim=128, dtype="bf16", backward=False),
}


def _graph(name, n, ss):
    """COO (src, dst) int64 for workload `name` at n nodes (n may be scaled down)."""
    meta = {}
    if name == "gt_uniform_n2708":
        m = int(round(10_556 * n / 2708))
        rng = np.random.default_rng(ss)
        idx = rng.choice(n * (n - 1), m, replace=False).astype(np.int64)
        u = idx // (n - 1)
        r = idx % (n - 1)
        v = r + (r >= u)
        src, dst = u, v
        src, dst = _relabel(ss.spawn(1)[0], n, src, dst)
    elif name in ("gt_chunglu25_n169k", "gt_chunglu22_n2450k"):
        if name == "gt_chunglu25_n169k":
            gamma, w_max, pairs = 2.5, 13_000.0, 1_170_000
            full = 169_343
        else:
            gamma, w_max, pairs = 2.2, 20_000.0, 62_000_000
            full = 2_450_000
        f = n / full
        k1, k2 = ss.spawn(2)
        src, dst, w = _chung_lu_pairs(k1, n, gamma, w_max * f, int(round(pairs * f)))
        meta["w_max"] = float(w[0])
        src, dst = _relabel(k2, n, src, dst)
    elif name == "gatv2_zipf21_n100k":
        k1, k2, k3 = ss.spawn(3)
        cap = max(1, int(round(50_000 * n / 100_000)))
        deg, s = zipf_in_degrees(k1, n, 2.1, 50.0, min(cap, n - 1))
        meta["zipf_scale"] = float(s)
        meta["mean_in_degree"] = float(deg.mean())
        src, dst = _distinct_sources(k2, n, deg, np.arange(n), np.ones(n, np.int64))
        src, dst = _relabel(k3, n, src, dst)
    elif name in ("gt_comm16_n1m_deg100", "gt_comm16_n1m_deg27"):
        if n % 16:
            raise ValueError("community workloads need n divisible by 16")
        inter = 84 if name.endswith("deg100") else 11
        c = np.arange(n // 16, dtype=np.int64)
        a, b = np.meshgrid(np.arange(16), np.arange(16), indexing="ij")
        off = (a != b)
        ia = a[off].ravel()
        ib = b[off].ravel()
        intra_src = (c[:, None] * 16 + ia[None, :]).ravel()
        intra_dst = (c[:, None] * 16 + ib[None, :]).ravel()
        node = np.arange(n, dtype=np.int64)
        isrc, idst = _distinct_sources(ss, n, np.full(n, inter, np.int64),
                                       (node // 16) * 16, np.full(n, 16, np.int64))
        src = np.concatenate([intra_src, isrc])
        dst = np.concatenate([intra_dst, idst])
    else:
        raise KeyError(name)
    return src.astype(np.int32), dst.astype(np.int32), meta


def make(name: str, n_nodes: Optional[int] = None, features: bool = True,
         backward: Optional[bool] = None) -> Workload:
    """Build workload `name` (see module doc). `n_nodes` scales the graph down
    with the same recipe (edge budgets, hub caps and w_max scale with n).
    `backward` overrides whether an upstream gradient dO is drawn."""
    spec = dict(SPECS[name])
    if backward is not None:
        spec["backward"] = bool(backward)
    n = int(n_nodes or spec["n"])
    root = np.random.SeedSequence([spec["seed"], n])
    g_ss, f_ss = root.spawn(2)
    src, dst, meta = _graph(spec.get("graph", name), n, g_ss)
    wl = Workload(name=name, kind=spec["kind"], n_nodes=n, src=src, dst=dst,
                  heads=spec["heads"], dim=spec["dim"], dtype=spec["dtype"],
                  backward=spec["backward"], seed=spec["seed"], meta=meta)
    if features:
        add_features(wl, f_ss)
    return wl


def add_features(wl: Workload, f_ss: Optional[np.random.SeedSequence] = None) -> None:
    if f_ss is None:
        f_ss = np.random.SeedSequence([wl.seed, wl.n_nodes]).spawn(2)[1]
    shape = (wl.n_nodes, wl.heads, wl.dim)
    names = {"gt": ["Q", "K", "V"], "gatv2": ["XD", "XS"], "reduce": ["X"], "spmm": ["X"]}[wl.kind]
    kids = f_ss.spawn(len(names) + 2)
    if wl.backward:
        names.append("dO")
    # the gradient stream is the last child so adding it leaves the others unchanged
    for nm, k in zip(names, list(kids[:len(names) - wl.backward]) + ([kids[-1]] if wl.backward else [])):
        if wl.dtype == "bf16":
            wl.bits[nm], wl.feats[nm] = normal_f32(k, shape, bf16=True)
        else:
            wl.feats[nm] = normal_f32(k, shape)
    if wl.kind == "gatv2":
        wl.att = normal_f32(kids[-2], (wl.heads, wl.dim), std=1.0 / np.sqrt(wl.dim))
