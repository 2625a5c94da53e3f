"""Pins for the oracle's summation scales and for the comparison function
every GPU parity test uses.

Each parity check passes when max_e |x_e - r_e| / max(|r_e|, S_e) is within
the tolerance, S_e being the oracle's condition scale of output e: the sum of
the absolute values of the terms reduced into it (SO, SL, SdQ, SdK, SdV for
the Graph Transformer; SdXD, SdXS, SdV, Sd_att for GATv2; S for SpMM). Those
scales are pinned here against values other than the oracle's own:
  * hand-worked examples (tests/golden/*scales*, gatv2_bwd_2node.txt,
    spmm_3node.txt) with mixed signs and cancelling outputs, so that a scale
    equal to |result|, a dropped weight or a dropped factor fails;
  * an independent dense computation (numpy, below) of every scale from the
    dense weight matrix;
and the comparison function itself is pinned on constructed arrays.
"""
import numpy as np
import pytest

import oracle
from _helpers import dense_adjacency, random_graph, read_golden


def _graph(seed, n, p=0.3):
    rng = np.random.default_rng(seed)
    src, dst, _ = random_graph(rng, n, p=p)
    ip, ix = oracle.csr_build(src, dst, n)
    return rng, ip, ix


def _close(a, b, tol=1e-13):
    a, b = np.asarray(a, np.float64).ravel(), np.asarray(b, np.float64).ravel()
    assert a.shape == b.shape
    return np.all(np.abs(a - b) <= tol * np.maximum(1.0, np.abs(b)))


# ------------------------------------------------------------ golden scales

def test_golden_gt_forward_scales():
    g = read_golden("gt_scales_3node.txt")
    N, H, D = int(g["N"][0]), int(g["H"][0]), int(g["D"][0])
    sh = (N, H, D)
    r = oracle.gt_fwd(g["indptr"].astype(np.int32), g["indices"].astype(np.int32), g["Q"].reshape(sh),
                      g["K"].reshape(sh), g["V"].reshape(sh))
    for k in ("O", "SO", "LSE", "SL"):
        assert _close(r[k], g[k]), k


def test_golden_gt_backward_scales():
    g = read_golden("gt_bwd_scales_2node.txt")
    N, H, D = int(g["N"][0]), int(g["H"][0]), int(g["D"][0])
    sh = (N, H, D)
    r = oracle.gt_bwd(g["indptr"].astype(np.int32), g["indices"].astype(np.int32), g["Q"].reshape(sh),
                      g["K"].reshape(sh), g["V"].reshape(sh), g["dO"].reshape(sh), scale=float(g["scale"][0]))
    for k in ("dQ", "dK", "dV", "Delta", "SdQ", "SdK", "SdV"):
        assert _close(r[k], g[k]), k
    # the same through the two halves the full-graph parity test calls
    ip, ix = g["indptr"].astype(np.int32), g["indices"].astype(np.int32)
    d = oracle.gt_bwd_dst(ip, ix, g["Q"].reshape(sh), g["K"].reshape(sh), g["V"].reshape(sh),
                          g["dO"].reshape(sh), scale=1.0)
    cip, cix = oracle.csc(ip, ix, N)
    s = oracle.gt_bwd_src(cip, cix, g["Q"].reshape(sh), g["K"].reshape(sh), g["V"].reshape(sh),
                          g["dO"].reshape(sh), d["M"], d["Z"], d["Delta"], scale=1.0)
    assert _close(d["SdQ"], g["SdQ"]) and _close(s["SdK"], g["SdK"]) and _close(s["SdV"], g["SdV"])


def test_golden_gatv2_backward_and_scales():
    g = read_golden("gatv2_bwd_2node.txt")
    N, H, D = int(g["N"][0]), int(g["H"][0]), int(g["D"][0])
    sh = (N, H, D)
    ip, ix = g["indptr"].astype(np.int32), g["indices"].astype(np.int32)
    att = g["att"].reshape(H, D)
    slope = float(g["slope"][0])
    f = oracle.gatv2_fwd(ip, ix, g["XD"].reshape(sh), g["XS"].reshape(sh), att, V=g["V"].reshape(sh),
                         slope=slope)
    assert _close(f["O"], g["O"]) and _close(f["LSE"], g["LSE"])
    r = oracle.gatv2_bwd(ip, ix, g["XD"].reshape(sh), g["XS"].reshape(sh), att, g["dO"].reshape(sh),
                         V=g["V"].reshape(sh), slope=slope)
    for k in ("Delta", "dXD", "SdXD", "dXS", "SdXS", "dV", "SdV", "d_att", "Sd_att"):
        assert _close(r[k], g[k]), k


def test_golden_spmm_scales():
    g = read_golden("spmm_3node.txt")
    N, F = int(g["N"][0]), int(g["F"][0])
    ip, ix = g["indptr"].astype(np.int32), g["indices"].astype(np.int32)
    X2 = g["X2"].reshape(N, F)
    r = oracle.spmm(ip, ix, X2, "gcn")
    assert _close(r["Y"], g["Y2_gcn"], 1e-15) and _close(r["S"], g["S2_gcn"], 1e-15)
    r = oracle.spmm(ip, ix, X2, "gcn", transpose=True)
    assert _close(r["Y"], g["YT2_gcn"], 1e-15) and _close(r["S"], g["ST2_gcn"], 1e-15)
    # with non-negative X the scale equals the result (sum of non-negative terms)
    X = g["X"].reshape(N, F)
    r = oracle.spmm(ip, ix, X, "gcn")
    assert _close(r["S"], g["Y_gcn"], 1e-15)


# ------------------------------------------------ dense independent scales

def _dense_softmax(S, A):
    S = np.where(A[None], S, -np.inf)
    m = S.max(axis=2, keepdims=True)
    m = np.where(np.isfinite(m), m, 0.0)
    P = np.exp(S - m)
    Z = P.sum(axis=2, keepdims=True)
    return np.divide(P, Z, out=np.zeros_like(P), where=Z > 0)


@pytest.mark.parametrize("seed,n,h,d", [(0, 20, 1, 16), (1, 33, 2, 8), (2, 17, 3, 5)])
def test_gt_scales_dense(seed, n, h, d):
    rng, ip, ix = _graph(seed, n)
    Q, K, V, dO = (rng.standard_normal((n, h, d)) for _ in range(4))
    sc = 1 / np.sqrt(d)
    A = dense_adjacency(ip, ix, n)
    S = sc * np.einsum("ihd,jhd->hij", Q, K)
    P = _dense_softmax(S, A)                                   # [h, i, j]
    SO = np.einsum("hij,jhd->ihd", P, np.abs(V))
    SL = 1 + np.where(A[None], np.abs(S), 0.0).max(axis=2).T
    dA = np.einsum("ihd,jhd->hij", dO, V)
    Dl = (P * dA).sum(axis=2)                                  # [h, i]
    Cm = P * (np.abs(dA) + np.abs(Dl)[:, :, None])             # zero off the graph (P = 0)
    SdQ = sc * np.einsum("hij,jhd->ihd", Cm, np.abs(K))
    SdK = sc * np.einsum("hij,ihd->jhd", Cm, np.abs(Q))
    SdV = np.einsum("hij,ihd->jhd", P, np.abs(dO))
    f = oracle.gt_fwd(ip, ix, Q, K, V)
    b = oracle.gt_bwd(ip, ix, Q, K, V, dO)
    for name, got, want in (("SO", f["SO"], SO), ("SL", f["SL"], SL), ("SdQ", b["SdQ"], SdQ),
                            ("SdK", b["SdK"], SdK), ("SdV", b["SdV"], SdV)):
        assert _close(got, want, 1e-12), name


@pytest.mark.parametrize("sep_v", [False, True])
@pytest.mark.parametrize("seed,n,h,d,slope", [(3, 15, 1, 4, 0.2), (4, 22, 2, 8, 0.05)])
def test_gatv2_scales_dense(seed, n, h, d, slope, sep_v):
    rng, ip, ix = _graph(seed, n)
    XD, XS, V, dO = (rng.standard_normal((n, h, d)) for _ in range(4))
    att = rng.standard_normal((h, d))
    Vv = V if sep_v else XS
    A = dense_adjacency(ip, ix, n)
    Zs = XS[None, :, :, :] + XD[:, None, :, :]                 # [i, j, h, d]
    phi = np.where(Zs >= 0, Zs, slope * Zs)
    dphi = np.where(Zs >= 0, 1.0, slope)
    S = np.einsum("ijhd,hd->hij", phi, att)
    P = _dense_softmax(S, A)
    dA = np.einsum("ihd,jhd->hij", dO, Vv)
    Dl = (P * dA).sum(axis=2)
    Cm = P * (np.abs(dA) + np.abs(Dl)[:, :, None])
    w = np.abs(att[None, None] * dphi)                         # |a phi'(z)| [i, j, h, d]
    SdXD = np.einsum("hij,ijhd->ihd", Cm, w)
    SdXS = np.einsum("hij,ijhd->jhd", Cm, w)
    SdV = np.einsum("hij,ihd->jhd", P, np.abs(dO))
    Sda = np.einsum("hij,ijhd->hd", Cm, np.abs(phi))
    r = oracle.gatv2_bwd(ip, ix, XD, XS, att, dO, V=V if sep_v else None, slope=slope)
    assert _close(r["SdXD"], SdXD, 1e-12)
    assert _close(r["Sd_att"], Sda, 1e-12)
    if sep_v:
        assert _close(r["SdXS"], SdXS, 1e-12) and _close(r["SdV"], SdV, 1e-12)
    else:
        assert _close(r["SdXS"], SdXS + SdV, 1e-12)
    f = oracle.gatv2_fwd(ip, ix, XD, XS, att, V=V if sep_v else None, slope=slope)
    assert _close(f["SO"], np.einsum("hij,jhd->ihd", P, np.abs(Vv)), 1e-12)
    assert _close(f["SL"], 1 + np.where(A[None], np.abs(S), 0.0).max(axis=2).T, 1e-12)


def test_scales_of_empty_rows():
    """A row without entries: O = 0 with SO = 0, LSE = -inf with SL = 1, and
    zero gradients with zero scales."""
    n, h, d = 5, 1, 4
    rng = np.random.default_rng(3)
    ip, ix = oracle.csr_build(np.array([1, 2], np.int32), np.array([0, 0], np.int32), n, add_self_loops=False)
    Q, K, V, dO = (rng.standard_normal((n, h, d)) for _ in range(4))
    f = oracle.gt_fwd(ip, ix, Q, K, V)
    b = oracle.gt_bwd(ip, ix, Q, K, V, dO)
    assert np.all(f["SO"][1:] == 0) and np.all(f["SL"][1:] == 1.0)
    assert np.all(b["SdQ"][1:] == 0)
    assert np.all(b["SdK"][[0, 3, 4]] == 0) and np.all(b["SdV"][[0, 3, 4]] == 0)


# ----------------------------------------------------- comparison function

def test_scaled_error_is_max_over_elements():
    ref = np.array([1.0, -2.0, 0.5, 0.0])
    S = np.array([0.1, 10.0, 4.0, 0.25])
    x = ref + np.array([0.01, 0.5, 0.0, -0.05])
    # per element: 0.01 / max(1, 0.1), 0.5 / max(2, 10), 0, 0.05 / max(0, 0.25)
    per = [0.01, 0.05, 0.0, 0.2]
    assert oracle.scaled_error(x, ref, S) == pytest.approx(max(per), rel=1e-12)
    assert oracle.scaled_error(x, ref, S) != pytest.approx(np.mean(per), rel=1e-3)
    # the reference's own magnitude is used where it exceeds the scale
    assert oracle.scaled_error([3.0], [2.0], [0.5]) == pytest.approx(0.5)
    # and the scale where it exceeds the magnitude
    assert oracle.scaled_error([2.1], [2.0], [20.0]) == pytest.approx(0.005)
    # exact agreement, and a broadcast scalar scale
    assert oracle.scaled_error(ref, ref, S) == 0.0
    assert oracle.scaled_error(x[:2], ref[:2], 10.0) == pytest.approx(0.05)
    # shapes beyond 1-D reduce over every element
    assert oracle.scaled_error(x.reshape(2, 2), ref.reshape(2, 2), S.reshape(2, 2)) == pytest.approx(0.2)
    assert oracle.scaled_error(np.zeros(0), np.zeros(0), np.zeros(0)) == 0.0


def test_scaled_error_infinities_and_nan():
    tol = 1e-4
    # empty rows' LSE: -inf on both sides is exact
    assert oracle.scaled_error([-np.inf, 1.0], [-np.inf, 1.0], [1.0, 1.0]) == 0.0
    assert oracle.scaled_error([np.inf], [np.inf], [1.0]) == 0.0
    # an infinity on one side only, or of the other sign, fails
    assert not oracle.scaled_error([0.0], [-np.inf], [1.0]) <= tol
    assert not oracle.scaled_error([-np.inf], [0.0], [1.0]) <= tol
    assert not oracle.scaled_error([np.inf], [-np.inf], [1.0]) <= tol
    # NaN anywhere fails the bar (the comparison with the tolerance is false)
    assert not oracle.scaled_error([np.nan, 1.0], [0.5, 1.0], [1.0, 1.0]) <= tol
    assert not oracle.scaled_error([1.0, 2.0], [1.0, np.nan], [1.0, 1.0]) <= tol


def test_normwise_error():
    ref = np.array([[1.0, -4.0], [2.0, 0.0]])
    x = ref + np.array([[0.0, 0.2], [-0.1, 0.4]])
    assert oracle.normwise_error(x, ref) == pytest.approx(0.4 / 4.0)
    assert oracle.normwise_error(ref, ref) == 0.0
    # non-finite reference entries (empty rows' LSE) are left out
    assert oracle.normwise_error([-np.inf, 1.5], [-np.inf, 1.0]) == pytest.approx(0.5)
    assert oracle.normwise_error([0.0], [0.0]) == 0.0
    assert oracle.normwise_error([1e-3], [0.0]) == np.inf
