"""Pins of the reduction-layer oracle (neighbourhood max / min of per-edge
messages with the winning source, and its gradient) against things other
than itself: a hand-worked example, an independent brute force, torch's
scatter_reduce and autograd, closed forms and invariants.

Source: "On Efficient Scaling of GNNs via IO-Aware Layers Implementations",
technical summary, Methodology (reduction-based aggregations: a per-edge
computation followed by a neighbourhood min/max)."""
import numpy as np
import pytest
import torch

import oracle
from _helpers import random_graph, read_golden


def _csr(src, dst, n):
    return oracle.csr_build(src, dst, n, add_self_loops=False)


def _brute(indptr, indices, X, op, msg):
    """Independent brute force: Python floats, an explicit key per candidate."""
    n, F = X.shape
    out = np.zeros((n, F), np.float32)
    arg = np.full((n, F), -1, np.int32)
    for i in range(n):
        ents = indices[indptr[i]:indptr[i + 1]]
        for f in range(F):
            cands = []
            for j in ents:
                m = np.float32(X[j, f]) - np.float32(X[i, f]) if msg == "diff" else np.float32(X[j, f])
                cands.append((float(m), int(j)))
            if not cands:
                continue
            if op == "max":
                v, j = max(cands, key=lambda c: (c[0], -c[1]))
            else:
                v, j = min(cands, key=lambda c: (c[0], c[1]))
            out[i, f] = v
            arg[i, f] = j
    return out, arg


def _same_bits(a, b):
    a = np.ascontiguousarray(a, np.float32)
    b = np.ascontiguousarray(b, np.float32)
    return np.array_equal(a.view(np.uint32), b.view(np.uint32))


def test_golden_4node():
    g = read_golden("reduce_4node.txt")
    n, F = int(g["N"][0]), int(g["F"][0])
    ip = g["indptr"].astype(np.int64)
    ix = g["indices"].astype(np.int32)
    X = g["X"].reshape(n, F).astype(np.float32)
    for op in ("max", "min"):
        for msg in ("src", "diff"):
            r = oracle.segment_reduce(ip, ix, X, op, msg)
            assert _same_bits(r["out"], g[f"{op}_{msg}_out"].reshape(n, F)), (op, msg)   # signs of zero too
            assert np.array_equal(r["arg"], g[f"{op}_{msg}_arg"].reshape(n, F).astype(np.int32)), (op, msg)
    dOut = g["dOut"].reshape(n, F)
    for msg in ("src", "diff"):
        arg = oracle.segment_reduce(ip, ix, X, "max", msg)["arg"]
        dX = oracle.segment_reduce_bwd(ip, ix, dOut, arg, msg)
        assert np.array_equal(dX, g[f"dX_max_{msg}"].reshape(n, F)), msg


@pytest.mark.parametrize("op", ["max", "min"])
@pytest.mark.parametrize("msg", ["src", "diff"])
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_brute_force_with_ties(op, msg, seed):
    """Small graphs with many ties (values drawn from a few levels, signed
    zeros included), duplicate entries and empty rows."""
    rng = np.random.default_rng(100 + seed)
    n, F = 30, 5
    src, dst, _ = random_graph(rng, n, p=0.2, self_loops=False)
    extra = rng.integers(0, n, (40, 2))              # duplicates survive: the CSR here keeps them
    src = np.concatenate([src, extra[:, 0]]).astype(np.int32)
    dst = np.concatenate([dst, extra[:, 1]]).astype(np.int32)
    keep = (dst != 0) & (dst != 7)                     # rows 0 and 7 empty
    src, dst = src[keep], dst[keep]
    order = np.lexsort((src, dst))
    src, dst = src[order], dst[order]
    indptr = np.concatenate([[0], np.cumsum(np.bincount(dst, minlength=n))]).astype(np.int64)
    indices = src.astype(np.int32)
    X = rng.choice(np.array([-1.5, -0.0, 0.0, 0.5, 2.0], np.float32), (n, F))
    assert (np.diff(indptr) == 0).any() and (np.diff(indices)[np.diff(indices) == 0].size > 0)
    r = oracle.segment_reduce(indptr, indices, X, op, msg)
    out, arg = _brute(indptr, indices, X, op, msg)
    assert np.array_equal(r["arg"], arg)
    assert _same_bits(r["out"], out)


@pytest.mark.parametrize("op,red", [("max", "amax"), ("min", "amin")])
def test_torch_scatter_reduce(op, red):
    """Values against torch's scatter_reduce (include_self=False keeps empty rows at 0)."""
    rng = np.random.default_rng(7)
    n, F = 200, 16
    src, dst, _ = random_graph(rng, n, p=0.05, self_loops=True)
    ip, ix = _csr(src, dst, n)
    X = rng.standard_normal((n, F)).astype(np.float32)
    r = oracle.segment_reduce(ip, ix, X, op, "src")
    deg = np.diff(ip)
    rows = np.repeat(np.arange(n), deg)
    ref = torch.zeros(n, F).scatter_reduce(0, torch.from_numpy(rows)[:, None].expand(-1, F),
                                           torch.from_numpy(X[ix]), reduce=red, include_self=False)
    assert np.array_equal(r["out"], ref.numpy())


def test_closed_forms():
    rng = np.random.default_rng(3)
    n, F = 60, 3
    src, dst, _ = random_graph(rng, n, p=0.1, self_loops=False)
    ip, ix = _csr(src, dst, n)
    deg = np.diff(ip)
    nz = deg > 0
    # X[j] = j: the max comes from the largest source, the min from the smallest
    Xj = np.repeat(np.arange(n, dtype=np.float32)[:, None], F, 1)
    mx = oracle.segment_reduce(ip, ix, Xj, "max")
    mn = oracle.segment_reduce(ip, ix, Xj, "min")
    last = np.array([ix[ip[i + 1] - 1] if deg[i] else -1 for i in range(n)])
    first = np.array([ix[ip[i]] if deg[i] else -1 for i in range(n)])
    assert np.array_equal(mx["arg"][:, 0], last) and np.array_equal(mn["arg"][:, 0], first)
    assert np.array_equal(mx["out"][nz, 0], last[nz].astype(np.float32))
    # constant X: every entry ties, the smallest source wins; diff messages are all +0
    Xc = np.full((n, F), 1.25, np.float32)
    for op in ("max", "min"):
        r = oracle.segment_reduce(ip, ix, Xc, op)
        assert np.array_equal(r["arg"][:, 1], first)
        assert np.all(r["out"][nz] == 1.25) and np.all(r["out"][~nz] == 0)
        d = oracle.segment_reduce(ip, ix, Xc, op, "diff")
        assert np.array_equal(d["arg"][:, 2], first) and not np.signbit(d["out"]).any()
    # empty rows: 0 and -1
    X = rng.standard_normal((n, F)).astype(np.float32)
    r = oracle.segment_reduce(ip, ix, X, "max")
    assert np.all(r["arg"][~nz] == -1) and np.all(r["out"][~nz] == 0)
    # diff values: the fp32 subtraction is monotone in x_j, so max_j (x_j - x_i) = (max_j x_j) - x_i
    d = oracle.segment_reduce(ip, ix, X, "max", "diff")
    assert np.array_equal(d["out"][nz], (r["out"] - X)[nz])
    dmin = oracle.segment_reduce(ip, ix, X, "min", "diff")
    rmin = oracle.segment_reduce(ip, ix, X, "min")
    assert np.array_equal(dmin["out"][nz], (rmin["out"] - X)[nz])


def test_invariants():
    rng = np.random.default_rng(4)
    n, F = 80, 6
    src, dst, _ = random_graph(rng, n, p=0.08, self_loops=True)
    ip, ix = _csr(src, dst, n)
    X = rng.standard_normal((n, F)).astype(np.float32)   # continuous: no ties
    mx = oracle.segment_reduce(ip, ix, X, "max")
    mn = oracle.segment_reduce(ip, ix, -X, "min")
    assert np.array_equal(mx["arg"], mn["arg"]) and np.array_equal(mx["out"], -mn["out"])
    # permutation equivariance: relabel node i as p[i]
    p = rng.permutation(n)
    ip2, ix2 = _csr(p[src].astype(np.int32), p[dst].astype(np.int32), n)
    X2 = np.empty_like(X)
    X2[p] = X
    for msg in ("src", "diff"):
        a = oracle.segment_reduce(ip, ix, X, "max", msg)
        b = oracle.segment_reduce(ip2, ix2, X2, "max", msg)
        assert np.array_equal(b["out"][p], a["out"])
        assert np.array_equal(b["arg"][p], np.where(a["arg"] >= 0, p[np.maximum(a["arg"], 0)], -1))
    # row subsets reproduce the full result
    rows = np.array([5, 0, 79, 33])
    sub = oracle.segment_reduce(ip, ix, X, "min", "diff", rows=rows)
    full = oracle.segment_reduce(ip, ix, X, "min", "diff")
    assert np.array_equal(sub["out"], full["out"][rows]) and np.array_equal(sub["arg"], full["arg"][rows])


@pytest.mark.parametrize("op,red", [("max", "amax"), ("min", "amin")])
@pytest.mark.parametrize("msg", ["src", "diff"])
def test_backward_torch_autograd(op, red, msg):
    """Gradient against torch autograd through the messages and scatter_reduce
    (continuous inputs, so no ties and the reduction is differentiable)."""
    rng = np.random.default_rng(11)
    n, F = 120, 8
    src, dst, _ = random_graph(rng, n, p=0.06, self_loops=True)
    ip, ix = _csr(src, dst, n)
    X = rng.standard_normal((n, F))
    dOut = rng.standard_normal((n, F))
    arg = oracle.segment_reduce(ip, ix, X.astype(np.float32), op, msg)["arg"]
    dX = oracle.segment_reduce_bwd(ip, ix, dOut, arg, msg)
    deg = np.diff(ip)
    rows = torch.from_numpy(np.repeat(np.arange(n), deg))
    Xt = torch.tensor(X, dtype=torch.float64, requires_grad=True)
    m = Xt[torch.from_numpy(ix.astype(np.int64))]
    if msg == "diff":
        m = m - Xt[rows]
    out = torch.zeros(n, F, dtype=torch.float64).scatter_reduce(0, rows[:, None].expand(-1, F), m, reduce=red,
                                                                  include_self=False)
    (out * torch.from_numpy(dOut)).sum().backward()
    assert np.allclose(dX, Xt.grad.numpy(), rtol=0, atol=1e-12)


def test_backward_finite_differences():
    rng = np.random.default_rng(12)
    n, F = 25, 3
    src, dst, _ = random_graph(rng, n, p=0.2, self_loops=True)
    ip, ix = _csr(src, dst, n)
    X = rng.standard_normal((n, F)).astype(np.float32).astype(np.float64)
    dOut = rng.standard_normal((n, F))
    for msg in ("src", "diff"):
        arg = oracle.segment_reduce(ip, ix, X.astype(np.float32), "max", msg)["arg"]
        dX = oracle.segment_reduce_bwd(ip, ix, dOut, arg, msg)

        def loss(Y):
            # fp64 evaluation of the same reduction through the fixed winners' definition
            tot = 0.0
            for i in range(n):
                ents = ix[ip[i]:ip[i + 1]]
                if ents.size == 0:
                    continue
                m = Y[ents] - (Y[i] if msg == "diff" else 0.0)
                tot += float((m.max(0) * dOut[i]).sum())
            return tot

        h = 1e-6
        for (j, f) in [(0, 0), (3, 2), (n - 1, 1), (10, 0)]:
            Yp, Ym = X.copy(), X.copy()
            Yp[j, f] += h
            Ym[j, f] -= h
            fd = (loss(Yp) - loss(Ym)) / (2 * h)
            assert abs(fd - dX[j, f]) < 1e-6, (msg, j, f, fd, dX[j, f])


def test_backward_counts_a_repeated_source_once():
    ip = np.array([0, 3], np.int64)
    ix = np.array([0, 0, 0], np.int32)
    X = np.array([[2.0]], np.float32)
    arg = oracle.segment_reduce(ip, ix, X, "max")["arg"]
    assert arg.tolist() == [[0]]
    assert oracle.segment_reduce_bwd(ip, ix, np.array([[5.0]]), arg).tolist() == [[5.0]]


def test_round_bf16():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5, 1.0 + 2 ** -9], np.float32)
    # ties to even at 1 + 2^-8 (halfway between 1 and 1 + 2^-7): down to 1; 1 + 3*2^-8: up to 1 + 2^-6
    assert oracle.round_bf16(x).tolist() == [1.0, 1.0, 1.0 + 2 ** -6, -2.5, 1.0]
