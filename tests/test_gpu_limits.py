"""GPU parity at the size limits of the heavy path and of the row width,
default plan (T = 512, C = 512, W = 4).

Hub graph: node 0 hears from all 2^19 other nodes and node 1 sends to all of
them, so one destination row and one source column each hold 524,288
entries (256 chunk groups and a second merge pass over 256 partials per
head group, in both the forward and the source pass of the backward; ten
times the largest degree of the benchmark graphs); every other row has two
or three entries. Wide rows: H = 16, D = 128 fp32 (8 KiB per node, eight
head groups per node) on a hub graph of 20,000 leaves. Outputs are compared
with the oracle on the hubs and a seeded sample of the other rows; gradient
identities are checked on the full outputs."""
import numpy as np
import pytest

import oracle
from _gpu import TOL, check, dev_feat, dev_i32, host, rand_feats, say

pytestmark = [pytest.mark.gpu, pytest.mark.slow]


@pytest.fixture(scope="module")
def g():
    import io_aware_sparse_amd as g
    g.lib()
    return g


def _hub_graph(m):
    """Edges j -> 0 for j >= 1 and 1 -> i for i >= 2 (self-loops added by the CSR build)."""
    n = m + 1
    src = np.concatenate([np.arange(1, n), np.ones(n - 2, np.int64)]).astype(np.int32)
    dst = np.concatenate([np.zeros(n - 1, np.int64), np.arange(2, n)]).astype(np.int32)
    return src, dst, n


def _check(name, x, ref, scale, dtype):
    check(name, x, ref, scale, dtype, f" over {np.asarray(ref).shape[0]} rows")


def _setup(g, m, seed):
    src, dst, n = _hub_graph(m)
    rp, rx = oracle.csr_build(src, dst, n)
    ip, ix = g.gnn_csr_build(dev_i32(src), dev_i32(dst), n)
    assert np.array_equal(ip.cpu().numpy(), rp) and np.array_equal(ix.cpu().numpy(), rx)
    plan = g.gnn_plan_create(ip, ix, want_csc=True)
    d = g.gnn_plan_export(plan)
    say(f"  N={n} E={rx.size}: heavy {d['n_heavy']} groups {d['n_groups']}, "
        f"source side heavy {d['c_n_heavy']} groups {d['c_n_groups']}")
    assert d["n_groups"] >= m // 2048 and d["c_n_groups"] >= m // 2048     # C * W = 2048 entries per group
    rng = np.random.default_rng(seed)
    rows = np.unique(np.concatenate([[0, 1, 2, n - 1], rng.choice(n, 2000, replace=False)]))
    return n, rp, rx, ip, ix, plan, rng, rows


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_gt_half_million_entry_hubs(g, dtype):
    import torch
    H, D = 2, 16
    say(f"GT hubs of 524k entries, {dtype}")
    n, rp, rx, ip, ix, plan, rng, rows = _setup(g, 1 << 19, 5)
    cip, cix = oracle.csc(rp, rx, n)
    Q, K, V, dO = rand_feats(rng, n, H, D, dtype, k=4)
    q, k, v, go = (dev_feat(x, dtype) for x in (Q, K, V, dO))
    O, L = g.gnn_attn_fwd(plan, ip, ix, q, k, v)
    dq, dk, dv = g.gnn_attn_bwd(plan, ip, ix, q, k, v, O, go, L)
    torch.cuda.synchronize()
    ref = oracle.gt_fwd(rp, rx, Q, K, V, rows=rows)
    _check("O", host(O)[rows], ref["O"], ref["SO"], dtype)
    _check("LSE", host(L)[rows], ref["LSE"], ref["SL"], "f32")
    rb = oracle.gt_bwd(rp, rx, Q, K, V, dO, rows=rows, srcs=rows, csc_arrays=(cip, cix))
    _check("dQ", host(dq)[rows], rb["dQ"], rb["SdQ"], dtype)
    _check("dK", host(dk)[rows], rb["dK"], rb["SdK"], dtype)
    _check("dV", host(dv)[rows], rb["dV"], rb["SdV"], dtype)
    sdk = dk.double().sum(0).abs()
    sdv = (dv.double().sum(0) - go.double().sum(0)).abs()
    tol = 1e-4 if dtype == "f32" else 2e-2
    assert torch.all(sdk <= tol * dk.double().abs().sum(0) + 1e-6)
    assert torch.all(sdv <= tol * dv.double().abs().sum(0) + 1e-6)


def test_gatv2_half_million_entry_hubs(g):
    import torch
    H, D, dtype = 4, 16, "f32"
    say("GATv2 hubs of 524k entries")
    n, rp, rx, ip, ix, plan, rng, rows = _setup(g, 1 << 19, 6)
    cip, cix = oracle.csc(rp, rx, n)
    XD, XS, dO = rand_feats(rng, n, H, D, dtype, k=3)
    att = (rng.standard_normal((H, D)) / np.sqrt(D)).astype(np.float32)
    xd, xs, go = (dev_feat(x, dtype) for x in (XD, XS, dO))
    at = torch.from_numpy(att).cuda()
    O, L = g.gatv2_attn_fwd(plan, ip, ix, xd, xs, at, negative_slope=0.2)
    gxd, gxs, _, gda = g.gatv2_attn_bwd(plan, ip, ix, xd, xs, at, go, L)
    torch.cuda.synchronize()
    ref = oracle.gatv2_fwd(rp, rx, XD, XS, att, slope=0.2, rows=rows)
    _check("O", host(O)[rows], ref["O"], ref["SO"], dtype)
    rb = oracle.gatv2_bwd(rp, rx, XD, XS, att, dO, slope=0.2, rows=rows, srcs=rows, csc_arrays=(cip, cix),
                          want_da=False)
    _check("dXD", host(gxd)[rows], rb["dXD"], rb["SdXD"], dtype)
    _check("dXS", host(gxs)[rows], rb["dXS"], rb["SdXS"], dtype)
    assert torch.isfinite(gda).all()


def test_gt_wide_rows_with_hub(g):
    """H = 16, D = 128 fp32: eight head groups per node, hubs of 20,000 entries."""
    import torch
    H, D, dtype = 16, 128, "f32"
    say("GT wide rows (16 x 128 fp32) with 20k-entry hubs")
    n, rp, rx, ip, ix, plan, rng, rows = _setup(g, 20_000, 7)
    rows = rows[:600]
    cip, cix = oracle.csc(rp, rx, n)
    Q, K, V, dO = rand_feats(rng, n, H, D, dtype, k=4)
    q, k, v, go = (dev_feat(x, dtype) for x in (Q, K, V, dO))
    O, L = g.gnn_attn_fwd(plan, ip, ix, q, k, v)
    dq, dk, dv = g.gnn_attn_bwd(plan, ip, ix, q, k, v, O, go, L)
    torch.cuda.synchronize()
    ref = oracle.gt_fwd(rp, rx, Q, K, V, rows=rows)
    _check("O", host(O)[rows], ref["O"], ref["SO"], dtype)
    rb = oracle.gt_bwd(rp, rx, Q, K, V, dO, rows=rows, srcs=rows, csc_arrays=(cip, cix))
    _check("dQ", host(dq)[rows], rb["dQ"], rb["SdQ"], dtype)
    _check("dK", host(dk)[rows], rb["dK"], rb["SdK"], dtype)
    _check("dV", host(dv)[rows], rb["dV"], rb["SdV"], dtype)
