"""The dependency subgraph the large GPU tests hand to the oracle.

On graphs too large for the oracle's tables, sampled outputs are compared
with the oracle run on the subgraph of their dependencies (the sampled rows
and sources, every destination of a sampled source, and all entries of those
rows, relabelled in increasing order). This pins that shortcut: on random
multigraphs with hubs, empty rows and repeated entries, every family's
results at the sampled rows and sources equal the full-graph oracle's
exactly, and the closed-form stride graph of the edge-limit test equals the
CSR and transposed adjacency the oracle builds from its edge list."""
import numpy as np
import pytest

import oracle
from _helpers import dependency_subgraph, stride_dests, stride_rows


def _multigraph(rng, n):
    m = 6 * n
    src = np.concatenate([rng.integers(0, n, m), np.full(n // 3, 3), rng.integers(0, n, n // 3)])
    dst = np.concatenate([rng.integers(0, n, m), rng.integers(0, n, n // 3), np.full(n // 3, 7)])
    rp, rx = oracle.csr_build(src.astype(np.int32), dst.astype(np.int32), n, add_self_loops=False)
    # repeat some entries (a multigraph row lists a source more than once)
    reps = rng.random(rx.size) < 0.05
    rows = np.repeat(np.arange(n), np.diff(rp))
    rows = np.concatenate([rows, rows[reps]])
    cols = np.concatenate([rx, rx[reps]])
    o = np.lexsort((cols, rows))
    rows, cols = rows[o], cols[o]
    rp = np.concatenate([[0], np.cumsum(np.bincount(rows, minlength=n))]).astype(np.int64)
    return rp, cols.astype(np.int32)


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_subgraph_oracle_equals_full_oracle(seed):
    rng = np.random.default_rng(seed)
    n = 1500
    rp, rx = _multigraph(rng, n)
    assert np.any(np.diff(rp) == 0)                 # empty rows present
    cip, cix = oracle.csc(rp, rx, n)
    rows = np.unique(np.concatenate([rng.choice(n, 40, replace=False), [3, 7]]))
    srcs = np.unique(np.concatenate([rng.choice(n, 30, replace=False), [3, 7]]))
    s = dependency_subgraph(rp, rx, cip, cix, rows, srcs)
    U = s["U"]
    assert U.size < n
    H, D = 2, 8
    Q, K, V, dO = (rng.standard_normal((n, H, D)) for _ in range(4))
    full = oracle.gt_fwd(rp, rx, Q, K, V, rows=rows)
    sub = oracle.gt_fwd(s["sp"], s["sx"], Q[U], K[U], V[U], rows=s["rows"])
    for k in ("O", "LSE", "SO", "SL"):
        assert np.array_equal(full[k], sub[k]), k
    full = oracle.gt_bwd(rp, rx, Q, K, V, dO, rows=rows, srcs=srcs)
    sub = oracle.gt_bwd(s["sp"], s["sx"], Q[U], K[U], V[U], dO[U], rows=s["rows"], srcs=s["srcs"])
    for k in ("dQ", "SdQ", "dK", "SdK", "dV", "SdV"):
        assert np.array_equal(full[k], sub[k]), k
    att = rng.standard_normal((H, D))
    full = oracle.gatv2_bwd(rp, rx, Q, K, att, dO, rows=rows, srcs=srcs, want_da=False)
    sub = oracle.gatv2_bwd(s["sp"], s["sx"], Q[U], K[U], att, dO[U], rows=s["rows"], srcs=s["srcs"],
                           want_da=False)
    for k in ("dXD", "SdXD", "dXS", "SdXS"):
        assert np.array_equal(full[k], sub[k]), k
    X = rng.standard_normal((n, 16)).astype(np.float32)
    dOut = rng.standard_normal((n, 16))
    at = {int(v): r for r, v in enumerate(s["need"])}
    ri = np.array([at[int(v)] for v in s["rows"]])
    for op, msg in (("max", "src"), ("min", "diff")):
        f = oracle.segment_reduce(rp, rx, X, op, msg)
        b = oracle.segment_reduce(s["sp"], s["sx"], X[U], op, msg, rows=s["need"])
        assert np.array_equal(f["out"][rows], b["out"][ri])
        assert np.array_equal(f["arg"][rows], np.where(b["arg"][ri] >= 0, U[np.maximum(b["arg"][ri], 0)], -1))
        fd, fS = oracle.segment_reduce_bwd(rp, rx, dOut, f["arg"], msg, want_scale=True)
        bd, bS = oracle.segment_reduce_bwd(s["sp"], s["sx"], dOut[U][s["need"]], b["arg"], msg, n_nodes=U.size,
                                           want_scale=True, rows=s["need"])
        assert np.array_equal(fd[srcs], bd[s["srcs"]]) and np.array_equal(fS[srcs], bS[s["srcs"]])
    for tr, ids, sids in ((False, rows, s["rows"]), (True, srcs, s["srcs"])):
        f = oracle.spmm(rp, rx, X, "mean", transpose=tr, rows=ids)
        b = oracle.spmm(s["sp"], s["sx"], X[U], "mean", transpose=tr, rows=sids)
        assert np.allclose(f["Y"], b["Y"], rtol=0, atol=1e-12) and np.allclose(f["S"], b["S"], rtol=0, atol=1e-12)


def test_subgraph_keeps_every_destination_row_whole():
    """A sampled source's column in the subgraph lists exactly its
    destinations in the full graph, each with its full row."""
    rng = np.random.default_rng(9)
    n = 800
    rp, rx = _multigraph(rng, n)
    cip, cix = oracle.csc(rp, rx, n)
    srcs = rng.choice(n, 20, replace=False)
    s = dependency_subgraph(rp, rx, cip, cix, np.array([0]), srcs)
    U = s["U"]
    scp, scx = oracle.csc(s["sp"], s["sx"], U.size)
    for j, lj in zip(srcs, s["srcs"]):
        assert np.array_equal(U[scx[scp[lj]:scp[lj + 1]]], cix[cip[j]:cip[j + 1]])
        for i in np.unique(cix[cip[j]:cip[j + 1]]):
            li = np.searchsorted(U, i)
            assert np.array_equal(U[s["sx"][s["sp"][li]:s["sp"][li + 1]]], rx[rp[i]:rp[i + 1]])


def test_stride_graph_closed_form():
    """Rows (i + step k) mod n, k < deg, of the edge-limit graph at a small
    size: the closed form equals the oracle's CSR of the edge list and its
    transposed adjacency."""
    n, step, deg = 4096, 513, 46
    i = np.arange(n)
    k = np.arange(1, deg)
    dst = np.repeat(i, deg - 1)
    src = ((i[:, None] + step * k[None, :]) % n).ravel()
    rp, rx = oracle.csr_build(src.astype(np.int32), dst.astype(np.int32), n)
    assert np.array_equal(rp, np.arange(n + 1) * deg)
    assert np.array_equal(rx.reshape(n, deg), stride_rows(i, n, step, deg))
    cip, cix = oracle.csc(rp, rx, n)
    for j in range(0, n, 61):
        assert np.array_equal(np.sort(stride_dests(j, n, step, deg)), cix[cip[j]:cip[j + 1]])
