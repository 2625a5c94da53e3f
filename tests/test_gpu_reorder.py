"""GPU parity of graph reordering (gnn_reorder, gnn_permute_graph,
gnn_permute_rows) against the oracle: permutations and relabelled CSRs bit
for bit, row permutations exact, attention on a relabelled graph against the
oracle, and the full-size graphs."""
import numpy as np
import pytest

import oracle
import workloads
from _gpu import TOL, check, dev_feat, dev_i32, host, say
from _helpers import read_golden

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def g():
    import io_aware_sparse_amd as g
    g.lib()
    return g


def _graphs():
    rng = np.random.default_rng(31)
    out = {}
    # random graph with self-loops (one component mostly)
    n = 500
    ip, ix = oracle.csr_build(rng.integers(0, n, 3000), rng.integers(0, n, 3000), n)
    out["random"] = (ip, ix, n)
    # many components and isolated nodes, no self-loops
    n = 700
    src, dst = [], []
    for c in range(40):
        base = 10 * c
        k = int(rng.integers(2, 10))
        for _ in range(2 * k):
            a, b = rng.integers(0, k, 2)
            src.append(base + a)
            dst.append(base + b)
    ip, ix = oracle.csr_build(np.array(src), np.array(dst), n, add_self_loops=False)
    out["components"] = (ip, ix, n)
    # multigraph with reciprocal pairs and repeated entries (CSR built by hand)
    n = 300
    s = rng.integers(0, n, 1500)
    d = rng.integers(0, n, 1500)
    s = np.concatenate([s, d[:200], s[:100]])
    d = np.concatenate([d, s[:200], d[:100]])
    o = np.lexsort((s, d))
    ip = np.concatenate([[0], np.cumsum(np.bincount(d, minlength=n))]).astype(np.int32)
    out["multigraph"] = (ip, s[o].astype(np.int32), n)
    # long path with shuffled labels (many levels)
    n = 2000
    q = rng.permutation(n)
    ip, ix = oracle.csr_build(q[:-1], q[1:], n, add_self_loops=False)
    out["path"] = (ip, ix, n)
    gd = read_golden("reorder_7node.txt")
    out["golden"] = (gd["indptr"].astype(np.int32), gd["indices"].astype(np.int32), 7)
    return out


GRAPHS = _graphs()


@pytest.mark.parametrize("name", sorted(GRAPHS))
@pytest.mark.parametrize("method", ["degree", "rcm"])
def test_reorder_and_relabel_exact(g, name, method):
    ip, ix, n = GRAPHS[name]
    say(f"reorder {method} on {name}: N={n} E={ix.size}")
    ip_d, ix_d = dev_i32(ip), dev_i32(ix)
    perm = g.gnn_reorder(ip_d, ix_d, method)
    ref = oracle.reorder(ip, ix, n, method)
    assert np.array_equal(perm.cpu().numpy(), ref)
    nip, nix = g.gnn_permute_graph(ip_d, ix_d, perm)
    rip, rix = oracle.permute_graph(ip, ix, ref)
    assert np.array_equal(nip.cpu().numpy(), rip) and np.array_equal(nix.cpu().numpy(), rix)


def test_permute_rows_round_trip(g):
    import torch
    rng = np.random.default_rng(2)
    n = 1000
    perm = rng.permutation(n).astype(np.int32)
    X = torch.from_numpy(rng.standard_normal((n, 3, 8)).astype(np.float32)).cuda()
    p = dev_i32(perm)
    Y = g.gnn_permute_rows(X, p)
    assert torch.equal(Y.cpu(), X.cpu()[torch.from_numpy(perm).long()])
    Z = g.gnn_permute_rows(Y, p, back=True)
    assert torch.equal(Z, X)
    B = X.to(torch.bfloat16).reshape(n, 24)
    assert torch.equal(g.gnn_permute_rows(g.gnn_permute_rows(B, p), p, back=True), B)
    bad = dev_i32(np.concatenate([perm[:-1], perm[:1]]))           # a repeated id
    with pytest.raises(g.GnnError):
        g.gnn_permute_rows(X, bad)
    with pytest.raises(g.GnnError):
        g.gnn_permute_graph(dev_i32(np.arange(n + 1, dtype=np.int32) * 0), dev_i32(np.zeros(0, np.int32)), bad)


@pytest.mark.parametrize("method", ["degree", "rcm"])
def test_attention_on_relabelled_graph(g, method):
    """GT forward on the relabelled graph and features against the oracle on
    the same relabelled input, and mapped back onto the original rows."""
    import torch
    wl = workloads.make("gt_chunglu25_n169k", n_nodes=4000)
    n, H, D = wl.n_nodes, wl.heads, wl.dim
    ip, ix = oracle.csr_build(wl.src, wl.dst, n)
    ip_d, ix_d = dev_i32(ip), dev_i32(ix)
    perm = g.gnn_reorder(ip_d, ix_d, method)
    nip, nix = g.gnn_permute_graph(ip_d, ix_d, perm)
    q, k, v = (dev_feat(wl.feats[nm], "f32") for nm in ("Q", "K", "V"))
    qp, kp, vp = (g.gnn_permute_rows(t, perm) for t in (q, k, v))
    plan = g.gnn_plan_create(nip, nix)
    O, L = g.gnn_attn_fwd(plan, nip, nix, qp, kp, vp)
    Ob = g.gnn_permute_rows(O, perm, back=True)
    ref = oracle.gt_fwd(ip, ix, wl.feats["Q"], wl.feats["K"], wl.feats["V"])
    check(f"{method}: relabelled GT forward O", host(Ob), ref["O"], ref["SO"], "f32")


@pytest.mark.slow
@pytest.mark.parametrize("name", ["gatv2_zipf21_n100k", "gt_chunglu22_n2450k"])
def test_reorder_full_size(g, name):
    import torch
    wl = workloads.make(name, features=False)
    n = wl.n_nodes
    ip_d, ix_d = g.gnn_csr_build(torch.from_numpy(wl.src).cuda(), torch.from_numpy(wl.dst).cuda(), n)
    ip, ix = ip_d.cpu().numpy(), ix_d.cpu().numpy()
    deg = oracle.total_degree(ip, ix, n)
    pd = g.gnn_reorder(ip_d, ix_d, "degree").cpu().numpy()
    assert np.array_equal(pd, oracle.reorder(ip, ix, n, "degree"))
    pr = g.gnn_reorder(ip_d, ix_d, "rcm").cpu().numpy()
    say(f"full-size reorder {name}: N={n} E={ix.size}")
    if n <= 200_000:
        assert np.array_equal(pr, oracle.reorder(ip, ix, n, "rcm"))
    else:
        # properties: a permutation whose last entry (first visited) is the node of smallest (degree, id)
        assert np.array_equal(np.sort(pr), np.arange(n))
        assert pr[-1] == np.lexsort((np.arange(n), deg))[0]
    nip, nix = g.gnn_permute_graph(ip_d, ix_d, torch.from_numpy(pr).cuda())
    assert int(nip[-1].item()) == ix.size
    b0, b1 = oracle.bandwidth(ip, ix), oracle.bandwidth(nip.cpu().numpy(), nix.cpu().numpy())
    say(f"  bandwidth {b0} -> {b1} after RCM")


def test_rcm_loop_caps_on_a_long_path(g, monkeypatch):
    """A 10,000-node path with shuffled labels (diameter 9,999). Component
    labelling (hooking with pointer jumping) finishes within
    ceil(log2 N) + 8 = 22 sweeps: with the sweep cap set to that, the order
    still equals the oracle's bit for bit. A sweep cap of 3, or a level cap
    below the path's 9,999 search levels, returns GNN_ERR_UNSUPPORTED."""
    from io_aware_sparse_amd import GnnError
    rng = np.random.default_rng(33)
    n = 10_000
    q = rng.permutation(n)
    ip, ix = oracle.csr_build(q[:-1], q[1:], n)
    want = oracle.reorder(ip, ix, n, "rcm")
    ip_d, ix_d = dev_i32(ip), dev_i32(ix)
    monkeypatch.setenv("GNN_RCM_MAX_SWEEPS", str(int(np.ceil(np.log2(n))) + 8))
    got = g.gnn_reorder(ip_d, ix_d, "rcm")
    assert np.array_equal(got.cpu().numpy(), want)
    for var, cap in (("GNN_RCM_MAX_SWEEPS", "3"), ("GNN_RCM_MAX_LEVELS", "9998")):
        monkeypatch.delenv("GNN_RCM_MAX_SWEEPS", raising=False)
        monkeypatch.setenv(var, cap)
        with pytest.raises(GnnError) as e:
            g.gnn_reorder(ip_d, ix_d, "rcm")
        assert e.value.status == -2, (var, cap)
        say(f"RCM on a {n}-node path with {var}={cap}: GNN_ERR_UNSUPPORTED")
    monkeypatch.setenv("GNN_RCM_MAX_LEVELS", "9999")
    assert np.array_equal(g.gnn_reorder(ip_d, ix_d, "rcm").cpu().numpy(), want)
