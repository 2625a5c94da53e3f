"""Randomised pins of the oracle's attention (Hypothesis, derandomised so the
examples are the same on every run): small random multigraphs, empty rows
included, against an independent dense formulation in which a source listed
c times in a row weighs c * exp(s) in the softmax (what the CSR definition
gives an entry that repeats), H in {1, 2, 4}, D in {4, 8, 16}.

  * GT forward (O, LSE) and GATv2 forward against the dense numpy form;
  * GT backward (dQ, dK, dV) against torch.autograd through the dense form
    in fp64 (rows without entries: O = 0, LSE = -inf, no gradient)."""
import numpy as np
import torch
from hypothesis import given, settings, strategies as st

import oracle

SETTINGS = settings(max_examples=40, deadline=None, derandomize=True)


@st.composite
def graphs(draw):
    n = draw(st.integers(1, 24))
    h = draw(st.sampled_from([1, 2, 4]))
    d = draw(st.sampled_from([4, 8, 16]))
    rows = [sorted(draw(st.lists(st.integers(0, n - 1), min_size=0, max_size=60))) for _ in range(n)]
    seed = draw(st.integers(0, 2 ** 31 - 1))
    ip = np.concatenate([[0], np.cumsum([len(r) for r in rows])]).astype(np.int32)
    ix = np.asarray([j for r in rows for j in r], np.int32)
    return n, h, d, ip, ix, seed


def counts(ip, ix, n):
    C = np.zeros((n, n))
    for i in range(n):
        for j in ix[ip[i]:ip[i + 1]]:
            C[i, j] += 1
    return C


def dense_softmax(C, S):
    """Per head h: softmax over row i of S[h] weighted by the entry counts C."""
    has = C.sum(1) > 0
    Sm = np.where(C[None] > 0, S, -np.inf)
    m = np.where(has[None, :, None], Sm.max(axis=2, keepdims=True), 0.0)
    P = C[None] * np.exp(np.where(C[None] > 0, S - m, -np.inf))
    Z = P.sum(axis=2, keepdims=True)
    A = np.divide(P, Z, out=np.zeros_like(P), where=Z > 0)
    LSE = np.where(has[None], (m[..., 0] + np.log(np.where(Z[..., 0] > 0, Z[..., 0], 1.0))), -np.inf)
    return A, LSE.T


@SETTINGS
@given(graphs())
def test_gt_forward_on_random_multigraphs(case):
    n, h, d, ip, ix, seed = case
    rng = np.random.default_rng(seed)
    Q, K, V = (rng.standard_normal((n, h, d)) for _ in range(3))
    r = oracle.gt_fwd(ip, ix, Q, K, V)
    A, LSE = dense_softmax(counts(ip, ix, n), np.einsum("ihd,jhd->hij", Q, K) / np.sqrt(d))
    O = np.einsum("hij,jhd->ihd", A, V)
    assert np.max(np.abs(r["O"] - O)) < 1e-12
    fin = np.isfinite(LSE)
    assert np.array_equal(np.isfinite(r["LSE"]), fin) and np.all(r["LSE"][~fin] == -np.inf)
    assert np.max(np.abs(r["LSE"][fin] - LSE[fin]), initial=0.0) < 1e-12


@SETTINGS
@given(graphs(), st.sampled_from([0.0, 0.2, 1.0]))
def test_gatv2_forward_on_random_multigraphs(case, slope):
    n, h, d, ip, ix, seed = case
    rng = np.random.default_rng(seed)
    XD, XS = (rng.standard_normal((n, h, d)) for _ in range(2))
    att = rng.standard_normal((h, d)) / np.sqrt(d)
    r = oracle.gatv2_fwd(ip, ix, XD, XS, att, slope=slope)
    Zs = XS[None, :, :, :] + XD[:, None, :, :]
    S = np.einsum("ijhd,hd->hij", np.where(Zs >= 0, Zs, slope * Zs), att)
    A, LSE = dense_softmax(counts(ip, ix, n), S)
    assert np.max(np.abs(r["O"] - np.einsum("hij,jhd->ihd", A, XS))) < 1e-12
    fin = np.isfinite(LSE)
    assert np.max(np.abs(r["LSE"][fin] - LSE[fin]), initial=0.0) < 1e-12


@SETTINGS
@given(graphs())
def test_gt_backward_on_random_multigraphs(case):
    n, h, d, ip, ix, seed = case
    rng = np.random.default_rng(seed)
    Q, K, V, dO = (rng.standard_normal((n, h, d)) for _ in range(4))
    g = oracle.gt_bwd(ip, ix, Q, K, V, dO)
    C = torch.tensor(counts(ip, ix, n))
    q, k, v = (torch.tensor(x, requires_grad=True) for x in (Q, K, V))
    S = torch.einsum("ihd,jhd->hij", q, k) / np.sqrt(d)
    Sm = torch.where(C[None] > 0, S, torch.full_like(S, -torch.inf))
    has = (C.sum(1) > 0)[None, :, None]
    m = torch.where(has, Sm.amax(dim=2, keepdim=True), torch.zeros(()))
    P = C[None] * torch.exp(torch.where(C[None] > 0, S - m.detach(), torch.full_like(S, -torch.inf)))
    Z = P.sum(dim=2, keepdim=True)
    A = torch.where(has, P / torch.where(has, Z, torch.ones(())), torch.zeros(()))
    torch.einsum("hij,jhd->ihd", A, v).backward(torch.tensor(dO))
    for name, t in (("dQ", q), ("dK", k), ("dV", v)):
        assert np.max(np.abs(g[name] - t.grad.numpy())) < 1e-11, name
