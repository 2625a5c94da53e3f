"""Small shared test utilities: golden-file parsing and tiny random graphs.

Nothing here computes attention; the independent dense references live in
the test files that use them."""
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def read_golden(name):
    out = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            k, v = line.split(":", 1)
            out[k.strip()] = np.array([float(t) for t in v.split()])
    return out


def random_graph(rng, n, p=0.3, self_loops=True, min_deg=0):
    """Small random digraph as COO (src, dst); optional self-pairs included
    directly (the oracle's CSR builder dedupes them)."""
    a = rng.random((n, n)) < p
    if self_loops:
        np.fill_diagonal(a, True)
    for i in range(n):
        if a[i].sum() < min_deg:
            a[i, rng.choice(n, min_deg, replace=False)] = True
    dst, src = np.nonzero(a)            # a[i, j]: edge j -> i
    return src.astype(np.int32), dst.astype(np.int32), a


def dense_adjacency(indptr, indices, n):
    a = np.zeros((n, n), bool)
    for i in range(n):
        a[i, indices[indptr[i]:indptr[i + 1]]] = True
    return a


def dependency_subgraph(rp, rx, cip, cix, rows, srcs):
    """The part of a CSR graph that outputs at `rows` (destination side) and
    `srcs` (source side) depend on, relabelled in increasing id order so that
    in-row order is kept: every sampled row and source, every destination of
    a sampled source, and all entries of those rows ("need"); other rows are
    left empty. A sampled source's destinations then keep their full rows,
    which is all its gradient depends on. Returns dict U (sorted global ids),
    sp / sx (the relabelled CSR) and the local ids of rows, srcs and need."""
    rp = np.asarray(rp, np.int64)
    cip = np.asarray(cip, np.int64)
    srcs = np.asarray(srcs, np.int64)
    rows = np.asarray(rows, np.int64)
    need = np.unique(np.concatenate([rows, srcs] + [cix[cip[s]:cip[s + 1]] for s in srcs]).astype(np.int64))
    U = np.unique(np.concatenate([need] + [rx[rp[i]:rp[i + 1]] for i in need]).astype(np.int64))
    loc = np.searchsorted(U, need)
    deg = np.zeros(U.size, np.int64)
    deg[loc] = rp[need + 1] - rp[need]
    sp = np.concatenate([[0], np.cumsum(deg)])
    sx = np.empty(int(sp[-1]), np.int32)
    for i, li in zip(need, loc):
        sx[sp[li]:sp[li + 1]] = np.searchsorted(U, rx[rp[i]:rp[i + 1]])
    return dict(U=U, sp=sp, sx=sx, rows=np.searchsorted(U, rows), srcs=np.searchsorted(U, srcs), need=loc)


def stride_rows(ids, n, step, deg):
    """Rows of the stride graph (row i lists (i + step*k) mod n, k = 0 .. deg-1,
    step odd and n a power of two, so the entries are distinct), sorted, as an
    int32 [len(ids), deg] array."""
    ids = np.asarray(ids, np.int64)
    return np.sort((ids[:, None] + step * np.arange(deg)[None, :]) % n, axis=1).astype(np.int32)


def stride_dests(j, n, step, deg):
    """Every row of the stride graph that lists source j."""
    return (j - step * np.arange(deg)) % n
