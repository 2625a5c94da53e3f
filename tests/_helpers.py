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
