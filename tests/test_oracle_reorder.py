"""Pins of the graph-reordering oracle (degree order, reverse Cuthill-McKee,
relabelled CSR) against a hand-worked example, scipy's reverse_cuthill_mckee
where the two definitions coincide, and closed forms.

Source: "On Efficient Scaling of GNNs via IO-Aware Layers Implementations",
technical summary, Methodology (graph reordering and its effect on
neighbour-parallel and feature-parallel kernels)."""
import numpy as np
import pytest
import scipy.sparse as sp
from scipy.sparse.csgraph import reverse_cuthill_mckee

import oracle
from _helpers import read_golden


def test_golden_7node():
    g = read_golden("reorder_7node.txt")
    n = int(g["N"][0])
    ip, ix = g["indptr"].astype(np.int64), g["indices"].astype(np.int64)
    assert np.array_equal(oracle.total_degree(ip, ix, n), g["degree"])
    assert np.array_equal(oracle.reorder(ip, ix, n, "degree"), g["perm_degree"])
    p = oracle.reorder(ip, ix, n, "rcm")
    assert np.array_equal(p, g["perm_rcm"])
    nip, nix = oracle.permute_graph(ip, ix, p)
    assert np.array_equal(nip, g["new_indptr"]) and np.array_equal(nix, g["new_indices"])


def _simple_connected(rng, n, m):
    """Connected simple digraph with no reciprocal pairs or self-loops (each
    undirected edge once, oriented at random) and a unique minimum-degree
    node: a random spanning tree plus random extra edges, and a pendant node."""
    edges = set()
    perm = rng.permutation(n - 1)
    for k in range(1, n - 1):                       # spanning tree on nodes 0..n-2
        a, b = int(perm[k]), int(perm[rng.integers(0, k)])
        edges.add((min(a, b), max(a, b)))
    while len(edges) < m:
        a, b = rng.integers(0, n - 1, 2)
        if a != b:
            edges.add((int(min(a, b)), int(max(a, b))))
    e = np.array(sorted(edges))
    deg = np.bincount(e.ravel(), minlength=n)
    hub = int(np.argmax(deg[:n - 1]))
    e = np.vstack([e, [[hub, n - 1]]])             # node n-1: the only node of degree 1 ...
    flip = rng.random(len(e)) < 0.5
    src = np.where(flip, e[:, 1], e[:, 0])
    dst = np.where(flip, e[:, 0], e[:, 1])
    deg = np.bincount(np.concatenate([src, dst]), minlength=n)
    return src.astype(np.int32), dst.astype(np.int32), deg


@pytest.mark.parametrize("seed", range(6))
def test_rcm_against_scipy(seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(20, 400))
    while True:
        src, dst, deg = _simple_connected(rng, n, int(n * rng.uniform(1.2, 4)))
        if np.sum(deg == deg.min()) == 1:          # ... unless the tree already had leaves of degree 1
            break
        n += 1
    ip, ix = oracle.csr_build(src, dst, n, add_self_loops=False)
    A = sp.csr_matrix((np.ones(ix.size), ix, ip), shape=(n, n))
    ref = reverse_cuthill_mckee(A, symmetric_mode=False)
    assert np.array_equal(oracle.reorder(ip, ix, n, "rcm"), ref)


def test_closed_forms():
    # a path 0-1-2-...-9 stored with edges i -> i+1: Cuthill-McKee from an end walks the path
    n = 10
    src = np.arange(n - 1, dtype=np.int32)
    dst = src + 1
    ip, ix = oracle.csr_build(src, dst, n, add_self_loops=False)
    assert oracle.reorder(ip, ix, n, "rcm").tolist() == list(range(n - 1, -1, -1))
    # shuffled labels: RCM still yields bandwidth 1 on a path
    rng = np.random.default_rng(1)
    q = rng.permutation(n)
    ip2, ix2 = oracle.csr_build(q[src].astype(np.int32), q[dst].astype(np.int32), n, add_self_loops=False)
    p = oracle.reorder(ip2, ix2, n, "rcm")
    assert oracle.bandwidth(*oracle.permute_graph(ip2, ix2, p)) == 1
    # star: centre 0 with leaves 1..7 pointing at it; degree order puts the centre first
    src = np.arange(1, 8, dtype=np.int32)
    dst = np.zeros(7, np.int32)
    ip, ix = oracle.csr_build(src, dst, 8, add_self_loops=False)
    assert oracle.reorder(ip, ix, 8, "degree").tolist() == [0, 1, 2, 3, 4, 5, 6, 7]
    # RCM of the star: start at leaf 1, then the centre, then leaves 2..7; reversed
    assert oracle.reorder(ip, ix, 8, "rcm").tolist() == [7, 6, 5, 4, 3, 2, 0, 1]


@pytest.mark.parametrize("method", ["degree", "rcm"])
def test_permutation_and_relabelling(method):
    rng = np.random.default_rng(7)
    n = 300
    src = rng.integers(0, n, 1500).astype(np.int32)
    dst = rng.integers(0, n, 1500).astype(np.int32)
    ip, ix = oracle.csr_build(src, dst, n)
    p = oracle.reorder(ip, ix, n, method)
    assert np.array_equal(np.sort(p), np.arange(n))
    nip, nix = oracle.permute_graph(ip, ix, p)
    # the relabelled graph is the same graph: edge multiset maps through the permutation
    inv = np.empty(n, np.int64)
    inv[p] = np.arange(n)
    old = set(zip(np.repeat(np.arange(n), np.diff(ip)).tolist(), ix.tolist()))
    new = set(zip(np.repeat(np.arange(n), np.diff(nip)).tolist(), nix.tolist()))
    assert new == {(int(inv[a]), int(inv[b])) for a, b in old}
    assert np.all(np.diff(nix)[np.diff(np.repeat(np.arange(n), np.diff(nip))) == 0] >= 0)   # rows sorted
    # relabelling back restores the graph
    bip, bix = oracle.permute_graph(nip, nix, inv.astype(np.int32))
    assert np.array_equal(bip, ip) and np.array_equal(bix, ix)
    if method == "rcm":
        assert oracle.bandwidth(nip, nix) <= oracle.bandwidth(ip, ix)
