"""Pins of the SpMM-aggregation oracle (Y = A_w X with sum, mean or GCN
weights, and its transpose) against a hand-worked example, an independent
dense brute force, torch's sparse product, closed forms and the adjoint
identity.

Source: "On Efficient Scaling of GNNs via IO-Aware Layers Implementations",
technical summary, Methodology (SpMM-based convolutions such as GCN and
GraphConv; cached normalised weights and transposed adjacency)."""
import numpy as np
import pytest
import torch

import oracle
from _helpers import random_graph, read_golden


def test_golden_3node():
    g = read_golden("spmm_3node.txt")
    n, F = int(g["N"][0]), int(g["F"][0])
    ip, ix = g["indptr"].astype(np.int64), g["indices"].astype(np.int64)
    X = g["X"].reshape(n, F)
    assert np.allclose(oracle.spmm_weights(ip, ix, "gcn"), g["gcn_w"], rtol=1e-14, atol=0)
    for norm in ("gcn", "mean", "sum"):
        assert np.allclose(oracle.spmm(ip, ix, X, norm)["Y"], g[f"Y_{norm}"].reshape(n, F), rtol=1e-14, atol=1e-15)
    assert np.allclose(oracle.spmm(ip, ix, X, "gcn", transpose=True)["Y"], g["YT_gcn"].reshape(n, F),
                       rtol=1e-14, atol=1e-15)


def _dense(ip, ix, n, norm):
    """Brute force: the weighted adjacency filled entry by entry, plain loops."""
    deg = [ip[i + 1] - ip[i] for i in range(n)]
    A = np.zeros((n, n))
    for i in range(n):
        for e in range(ip[i], ip[i + 1]):
            j = ix[e]
            w = 1.0 if norm == "sum" else (1.0 / deg[i] if norm == "mean" else 1.0 / np.sqrt(deg[i] * deg[j]))
            A[i, j] += w
    return A


@pytest.mark.parametrize("norm", ["sum", "mean", "gcn"])
def test_dense_brute_force_and_transpose(norm):
    rng = np.random.default_rng(3)
    n, F = 40, 5
    src, dst, _ = random_graph(rng, n, p=0.15, self_loops=True)
    ip, ix = oracle.csr_build(src, dst, n)
    X = rng.standard_normal((n, F))
    A = _dense(ip, ix, n, norm)
    assert np.allclose(oracle.spmm(ip, ix, X, norm)["Y"], A @ X, rtol=0, atol=1e-13)
    assert np.allclose(oracle.spmm(ip, ix, X, norm, transpose=True)["Y"], A.T @ X, rtol=0, atol=1e-13)


def test_torch_sparse_and_repeats():
    rng = np.random.default_rng(4)
    n, F = 300, 16
    s = rng.integers(0, n, 2000)
    d = rng.integers(0, n, 2000)
    s = np.concatenate([s, s[:300], np.arange(n)])          # repeated entries and self-loops
    d = np.concatenate([d, d[:300], np.arange(n)])
    o = np.lexsort((s, d))
    ip = np.concatenate([[0], np.cumsum(np.bincount(d, minlength=n))]).astype(np.int64)
    ix = s[o]
    X = rng.standard_normal((n, F))
    # weights computed independently with torch ops
    rows = torch.from_numpy(np.repeat(np.arange(n), np.diff(ip)))
    cols = torch.from_numpy(ix)
    deg = torch.bincount(rows, minlength=n).double()
    w = 1.0 / torch.sqrt(deg[rows] * deg[cols])
    A = torch.sparse_coo_tensor(torch.stack([rows, cols]), w, (n, n)).coalesce()
    ref = torch.sparse.mm(A, torch.from_numpy(X)).numpy()
    assert np.allclose(oracle.spmm(ip, ix, X, "gcn")["Y"], ref, rtol=0, atol=1e-12)


def test_gcn_source_without_entries():
    # row 0 = {1}, row 1 empty: source 1 has no entries of its own, so its factor is 0 (no 1/sqrt(0))
    ip = np.array([0, 1, 1], np.int64)
    ix = np.array([1], np.int64)
    assert oracle.spmm_weights(ip, ix, "gcn").tolist() == [0.0]
    assert np.all(oracle.spmm(ip, ix, np.ones((2, 3)), "gcn")["Y"] == 0)
    assert oracle.spmm_weights(ip, ix, "mean").tolist() == [1.0]


def test_closed_forms_and_adjoint():
    rng = np.random.default_rng(5)
    n, F = 200, 4
    src, dst, _ = random_graph(rng, n, p=0.05, self_loops=True)
    ip, ix = oracle.csr_build(src, dst, n)
    ones = np.ones((n, F))
    assert np.allclose(oracle.spmm(ip, ix, ones, "mean")["Y"], 1.0, atol=1e-14)
    assert np.allclose(oracle.spmm(ip, ix, ones, "sum")["Y"][:, 0], np.diff(ip))
    # d-regular directed graph (circulant): gcn weights 1/d, rows of A_w sum to one
    d = 5
    src = (np.arange(n)[:, None] + np.arange(1, d)[None, :]).ravel() % n
    dst = np.repeat(np.arange(n), d - 1)
    ip2, ix2 = oracle.csr_build(src, dst, n)                 # plus self-loops: in-degree d everywhere
    assert np.allclose(oracle.spmm(ip2, ix2, ones, "gcn")["Y"], 1.0, atol=1e-14)
    # adjoint: <A X, Y> = <X, A^T Y>
    X = rng.standard_normal((n, F))
    Y = rng.standard_normal((n, F))
    for norm in ("sum", "mean", "gcn"):
        lhs = np.sum(oracle.spmm(ip, ix, X, norm)["Y"] * Y)
        rhs = np.sum(X * oracle.spmm(ip, ix, Y, norm, transpose=True)["Y"])
        assert abs(lhs - rhs) <= 1e-12 * max(1.0, abs(lhs))
    # the scale bounds the result
    r = oracle.spmm(ip, ix, X, "gcn")
    assert np.all(np.abs(r["Y"]) <= r["S"] + 1e-15)
