"""GPU parity of the fused attention kernels against the fp64 oracle.

Graphs are small enough for the oracle to finish in seconds but span many
workgroups, heavy rows with several chunk groups and ragged last chunks, and
rows whose degree is not a multiple of the per-step edge count. Plans are
exercised light-only, heavy-forced and mixed."""
import numpy as np
import pytest

import oracle
import workloads
from _gpu import TOL, check, dev_feat, dev_i32, host, rand_feats, say

pytestmark = pytest.mark.gpu

PLANS = {
    "none": None,
    "light": dict(light_threshold=10 ** 9, chunk=512, waves_per_group=4),
    "heavy": dict(light_threshold=0, chunk=5, waves_per_group=4),
    "heavy_w1": dict(light_threshold=0, chunk=3, waves_per_group=1),
    "mixed": dict(light_threshold=16, chunk=8, waves_per_group=2),
    "mixed_w8": dict(light_threshold=40, chunk=16, waves_per_group=8),
}


@pytest.fixture(scope="module")
def g():
    import io_aware_sparse_amd as g
    g.lib()
    return g


def _graph(g, seed, n, self_loops=True):
    """Chung-Lu power-law graph (hubs up to a few hundred in-edges)."""
    wl = workloads.make("gt_chunglu25_n169k", n, features=False)
    src, dst = wl.src, wl.dst
    if not self_loops:
        # drop every in-edge of a few nodes to create empty rows
        rng = np.random.default_rng(seed)
        empty = rng.choice(n, max(1, n // 50), replace=False)
        keep = ~np.isin(dst, empty)
        src, dst = src[keep], dst[keep]
    rp, rx = oracle.csr_build(src, dst, n, add_self_loops=self_loops)
    ip, ix = g.gnn_csr_build(dev_i32(src), dev_i32(dst), n, add_self_loops=self_loops)
    assert np.array_equal(ip.cpu().numpy(), rp) and np.array_equal(ix.cpu().numpy(), rx)
    return ip, ix, rp, rx


def _plan(g, ip, ix, name, want_csc=False):
    p = PLANS[name]
    return None if p is None else g.gnn_plan_create(ip, ix, want_csc=want_csc, **p)


def _check(name, x, ref, scale, dtype):
    check(name, x, ref, scale, dtype)


CASES = [("f32", 16, 1), ("f32", 32, 4), ("f32", 64, 2), ("f32", 128, 3), ("f32", 16, 8),
         ("bf16", 16, 2), ("bf16", 32, 4), ("bf16", 64, 8), ("bf16", 128, 1)]


@pytest.mark.parametrize("dtype,D,H", CASES)
@pytest.mark.parametrize("plan", ["none", "light", "heavy", "mixed"])
def test_gt_fwd_parity(g, dtype, D, H, plan):
    n = 3000
    say("gt_fwd", dtype, D, H, plan)
    ip, ix, rp, rx = _graph(g, 1, n)
    rng = np.random.default_rng(D * 7 + H)
    Q, K, V = rand_feats(rng, n, H, D, dtype)
    pl = _plan(g, ip, ix, plan)
    O, L = g.gnn_attn_fwd(pl, ip, ix, dev_feat(Q, dtype), dev_feat(K, dtype), dev_feat(V, dtype))
    ref = oracle.gt_fwd(rp, rx, Q, K, V)
    _check("O", host(O), ref["O"], ref["SO"], dtype)
    _check("LSE", host(L), ref["LSE"], ref["SL"], "f32")


@pytest.mark.parametrize("plan", ["none", "heavy_w1", "mixed", "mixed_w8"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_gt_fwd_empty_rows_and_scale(g, plan, dtype):
    n, H, D = 2500, 2, 32
    say("gt_fwd empty rows", plan, dtype)
    ip, ix, rp, rx = _graph(g, 2, n, self_loops=False)
    assert np.any(np.diff(rp) == 0)
    rng = np.random.default_rng(3)
    Q, K, V = rand_feats(rng, n, H, D, dtype)
    pl = _plan(g, ip, ix, plan)
    O, L = g.gnn_attn_fwd(pl, ip, ix, dev_feat(Q, dtype), dev_feat(K, dtype), dev_feat(V, dtype), scale=0.3)
    ref = oracle.gt_fwd(rp, rx, Q, K, V, scale=0.3)
    _check("O", host(O), ref["O"], ref["SO"], dtype)
    _check("LSE", host(L), ref["LSE"], ref["SL"], "f32")
    empty = np.diff(rp) == 0
    assert np.all(host(O)[empty] == 0) and np.all(np.isneginf(host(L)[empty]))


@pytest.mark.parametrize("dtype,D,H", [("f32", 32, 4), ("f32", 16, 8), ("bf16", 64, 4)])
@pytest.mark.parametrize("plan", ["heavy_w1", "mixed", "mixed_w8"])
def test_packed_light_rows_with_empty_rows(g, dtype, D, H, plan):
    """Rows of 257-512 bytes run two per wave from the descending-degree list:
    empty rows, an odd number of light rows (the last wave holds one row) and
    both attention modes against the oracle."""
    import torch
    n = 2501
    say("packed light rows", dtype, D, H, plan)
    ip, ix, rp, rx = _graph(g, 4, n, self_loops=False)
    empty = np.diff(rp) == 0
    assert empty.any()
    pl = _plan(g, ip, ix, plan)
    n_light = g.gnn_plan_export(pl)["n_light"]
    say(f"  light rows {n_light}, empty rows {int(empty.sum())}")
    rng = np.random.default_rng(5)
    Q, K, V = rand_feats(rng, n, H, D, dtype)
    q, k, v = (dev_feat(x, dtype) for x in (Q, K, V))
    O, L = g.gnn_attn_fwd(pl, ip, ix, q, k, v)
    ref = oracle.gt_fwd(rp, rx, Q, K, V)
    _check("O", host(O), ref["O"], ref["SO"], dtype)
    _check("LSE", host(L), ref["LSE"], ref["SL"], "f32")
    assert np.all(host(O)[empty] == 0) and np.all(np.isneginf(host(L)[empty]))
    att = (rng.standard_normal((H, D)) / np.sqrt(D)).astype(np.float32)
    Og, Lg = g.gatv2_attn_fwd(pl, ip, ix, q, k, torch.from_numpy(att).cuda())
    rg = oracle.gatv2_fwd(rp, rx, Q, K, att)
    _check("GATv2 O", host(Og), rg["O"], rg["SO"], dtype)
    _check("GATv2 LSE", host(Lg), rg["LSE"], rg["SL"], "f32")


@pytest.mark.parametrize("dtype,D,H", [("f32", 16, 8), ("f32", 32, 2), ("bf16", 16, 8), ("bf16", 64, 4),
                                       ("f32", 128, 1)])
@pytest.mark.parametrize("plan", ["none", "heavy", "mixed"])
@pytest.mark.parametrize("sep_v", [False, True])
def test_gatv2_fwd_parity(g, dtype, D, H, plan, sep_v):
    n = 3000
    say("gatv2_fwd", dtype, D, H, plan, sep_v)
    ip, ix, rp, rx = _graph(g, 4, n)
    rng = np.random.default_rng(D + H)
    XD, XS, V = rand_feats(rng, n, H, D, dtype)
    att = (rng.standard_normal((H, D)) / np.sqrt(D)).astype(np.float32)
    import torch
    pl = _plan(g, ip, ix, plan)
    xs = dev_feat(XS, dtype)
    O, L = g.gatv2_attn_fwd(pl, ip, ix, dev_feat(XD, dtype), xs, torch.from_numpy(att).cuda(),
                            V=dev_feat(V, dtype) if sep_v else None, negative_slope=0.2)
    ref = oracle.gatv2_fwd(rp, rx, XD, XS, att, V=V if sep_v else None, slope=0.2)
    _check("O", host(O), ref["O"], ref["SO"], dtype)
    _check("LSE", host(L), ref["LSE"], ref["SL"], "f32")


@pytest.mark.parametrize("dtype,D,H", [("f32", 16, 1), ("f32", 32, 4), ("f32", 64, 3), ("f32", 128, 2),
                                       ("bf16", 32, 4), ("bf16", 64, 8), ("bf16", 16, 2)])
@pytest.mark.parametrize("plan", ["light", "heavy", "mixed", "mixed_w8"])
def test_gt_bwd_parity(g, dtype, D, H, plan):
    n = 2500
    say("gt_bwd", dtype, D, H, plan)
    ip, ix, rp, rx = _graph(g, 5, n, self_loops=(plan != "mixed"))
    rng = np.random.default_rng(11 * D + H)
    Q, K, V, dO = rand_feats(rng, n, H, D, dtype, k=4)
    pl = _plan(g, ip, ix, plan, want_csc=True)
    q, k, v, go = (dev_feat(x, dtype) for x in (Q, K, V, dO))
    O, L = g.gnn_attn_fwd(pl, ip, ix, q, k, v)
    dq, dk, dv = g.gnn_attn_bwd(pl, ip, ix, q, k, v, O, go, L)
    ref = oracle.gt_bwd(rp, rx, Q, K, V, dO)
    _check("dQ", host(dq), ref["dQ"], ref["SdQ"], dtype)
    _check("dK", host(dk), ref["dK"], ref["SdK"], dtype)
    _check("dV", host(dv), ref["dV"], ref["SdV"], dtype)


def test_determinism_bitwise(g):
    n, H, D, dtype = 4000, 4, 32, "bf16"
    say("determinism")
    ip, ix, rp, rx = _graph(g, 6, n)
    rng = np.random.default_rng(6)
    q, k, v, go = (dev_feat(x, dtype) for x in rand_feats(rng, n, H, D, dtype, k=4))
    pl = _plan(g, ip, ix, "mixed", want_csc=True)
    outs = []
    for _ in range(2):
        O, L = g.gnn_attn_fwd(pl, ip, ix, q, k, v)
        dq, dk, dv = g.gnn_attn_bwd(pl, ip, ix, q, k, v, O, go, L)
        outs.append([t.clone() for t in (O, L, dq, dk, dv)])
    import torch
    for a, b in zip(*outs):
        assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a,
                           b.view(torch.int16) if b.dtype == torch.bfloat16 else b)


def test_special_graphs(g):
    import torch
    rng = np.random.default_rng(8)
    H, D, dtype = 2, 16, "f32"
    graphs = {}
    n = 700                                             # star: node 0 hears from everyone
    graphs["star"] = (np.arange(1, n, dtype=np.int32), np.zeros(n - 1, np.int32), n)
    n = 64                                              # complete digraph
    a, b = np.meshgrid(np.arange(n), np.arange(n))
    graphs["complete"] = (a.ravel().astype(np.int32), b.ravel().astype(np.int32), n)
    graphs["single"] = (np.zeros(0, np.int32), np.zeros(0, np.int32), 1)
    graphs["self_only"] = (np.zeros(0, np.int32), np.zeros(0, np.int32), 300)
    for name, (src, dst, n) in graphs.items():
        say("special", name)
        rp, rx = oracle.csr_build(src, dst, n)
        ip, ix = g.gnn_csr_build(dev_i32(src), dev_i32(dst), n)
        assert np.array_equal(ip.cpu().numpy(), rp) and np.array_equal(ix.cpu().numpy(), rx)
        Q, K, V, dO = rand_feats(rng, n, H, D, dtype, k=4)
        for plan in ("light", "heavy", "mixed"):
            pl = _plan(g, ip, ix, plan, want_csc=True)
            q, k, v, go = (dev_feat(x, dtype) for x in (Q, K, V, dO))
            O, L = g.gnn_attn_fwd(pl, ip, ix, q, k, v)
            ref = oracle.gt_fwd(rp, rx, Q, K, V)
            _check(f"{name}/{plan} O", host(O), ref["O"], ref["SO"], dtype)
            dq, dk, dv = g.gnn_attn_bwd(pl, ip, ix, q, k, v, O, go, L)
            rb = oracle.gt_bwd(rp, rx, Q, K, V, dO)
            _check(f"{name}/{plan} dQ", host(dq), rb["dQ"], rb["SdQ"], dtype)
            _check(f"{name}/{plan} dK", host(dk), rb["dK"], rb["SdK"], dtype)
            _check(f"{name}/{plan} dV", host(dv), rb["dV"], rb["SdV"], dtype)
    torch.cuda.synchronize()


def test_multigraph_rows(g):
    """Duplicate entries in a row are each counted (CSR assembled on the host)."""
    import torch
    n, H, D, dtype = 500, 2, 32, "f32"
    rng = np.random.default_rng(9)
    deg = rng.integers(0, 40, n)
    rp = np.concatenate([[0], np.cumsum(deg)]).astype(np.int32)
    rx = np.concatenate([np.sort(rng.integers(0, 20, d)) for d in deg]).astype(np.int32)  # many repeats
    ip, ix = dev_i32(rp), dev_i32(rx)
    Q, K, V, dO = rand_feats(rng, n, H, D, dtype, k=4)
    for plan in ("none", "heavy", "mixed"):
        say("multigraph", plan)
        pl = _plan(g, ip, ix, plan, want_csc=plan != "none")
        q, k, v, go = (dev_feat(x, dtype) for x in (Q, K, V, dO))
        O, L = g.gnn_attn_fwd(pl, ip, ix, q, k, v)
        ref = oracle.gt_fwd(rp, rx, Q, K, V)
        _check("O", host(O), ref["O"], ref["SO"], dtype)
        if pl is not None:
            dq, dk, dv = g.gnn_attn_bwd(pl, ip, ix, q, k, v, O, go, L)
            rb = oracle.gt_bwd(rp, rx, Q, K, V, dO)
            _check("dK", host(dk), rb["dK"], rb["SdK"], dtype)
            _check("dV", host(dv), rb["dV"], rb["SdV"], dtype)
    torch.cuda.synchronize()


def test_gpu_identities(g):
    """Properties that hold for any size, checked on GPU outputs."""
    import torch
    n, H, D, dtype = 6000, 4, 32, "f32"
    say("identities")
    ip, ix, rp, rx = _graph(g, 10, n)
    rng = np.random.default_rng(10)
    Q, K, V, dO = rand_feats(rng, n, H, D, dtype, k=4)
    pl = _plan(g, ip, ix, "mixed", want_csc=True)
    q, k, v, go = (dev_feat(x, dtype) for x in (Q, K, V, dO))
    # V constant -> O constant
    O1, _ = g.gnn_attn_fwd(pl, ip, ix, q, k, torch.full_like(v, 0.75))
    assert torch.max(torch.abs(O1 - 0.75)).item() < 1e-5
    O, L = g.gnn_attn_fwd(pl, ip, ix, q, k, v)
    dq, dk, dv = g.gnn_attn_bwd(pl, ip, ix, q, k, v, O, go, L)
    # shift invariance: sum of dK over sources vanishes; weights sum to one:
    # sum of dV over sources equals the sum of dO over destinations
    sdk = dk.double().sum(0).abs()
    sdv = (dv.double().sum(0) - go.double().sum(0)).abs()
    assert torch.all(sdk <= 1e-4 * dk.double().abs().sum(0) + 1e-6)
    assert torch.all(sdv <= 1e-4 * dv.double().abs().sum(0) + 1e-6)


@pytest.mark.parametrize("dtype,D,H", [("f32", 16, 8), ("f32", 32, 2), ("f32", 128, 1), ("bf16", 16, 8),
                                       ("bf16", 64, 4), ("bf16", 32, 3)])
@pytest.mark.parametrize("plan", ["light", "heavy", "mixed", "mixed_w8"])
@pytest.mark.parametrize("sep_v", [False, True])
def test_gatv2_bwd_parity(g, dtype, D, H, plan, sep_v):
    import torch
    n = 2500
    say("gatv2_bwd", dtype, D, H, plan, sep_v)
    ip, ix, rp, rx = _graph(g, 12, n, self_loops=(plan != "mixed"))
    rng = np.random.default_rng(7 * D + H)
    XD, XS, V, dO = rand_feats(rng, n, H, D, dtype, k=4)
    att = (rng.standard_normal((H, D)) / np.sqrt(D)).astype(np.float32)
    pl = _plan(g, ip, ix, plan, want_csc=True)
    xd, xs, v, go = (dev_feat(x, dtype) for x in (XD, XS, V, dO))
    a = torch.from_numpy(att).cuda()
    O, L = g.gatv2_attn_fwd(pl, ip, ix, xd, xs, a, V=v if sep_v else None)
    gxd, gxs, gv, gda = g.gatv2_attn_bwd(pl, ip, ix, xd, xs, a, go, L, V=v if sep_v else None)
    ref = oracle.gatv2_bwd(rp, rx, XD, XS, att, dO, V=V if sep_v else None, slope=0.2)
    _check("dXD", host(gxd), ref["dXD"], ref["SdXD"], dtype)
    _check("dXS", host(gxs), ref["dXS"], ref["SdXS"], dtype)
    if sep_v:
        _check("dV", host(gv), ref["dV"], ref["SdV"], dtype)
    _check("d_att", gda.cpu().numpy(), ref["d_att"], ref["Sd_att"], dtype)


def test_gatv2_bwd_deterministic(g):
    import torch
    n, H, D, dtype = 3000, 8, 16, "f32"
    ip, ix, rp, rx = _graph(g, 13, n)
    rng = np.random.default_rng(13)
    xd, xs, go = (dev_feat(x, dtype) for x in rand_feats(rng, n, H, D, dtype, k=3))
    a = torch.from_numpy((rng.standard_normal((H, D)) / 4).astype(np.float32)).cuda()
    pl = _plan(g, ip, ix, "mixed", want_csc=True)
    O, L = g.gatv2_attn_fwd(pl, ip, ix, xd, xs, a)
    r1 = [t.clone() for t in g.gatv2_attn_bwd(pl, ip, ix, xd, xs, a, go, L) if t is not None]
    r2 = [t.clone() for t in g.gatv2_attn_bwd(pl, ip, ix, xd, xs, a, go, L) if t is not None]
    for x, y in zip(r1, r2):
        assert torch.equal(x, y)


@pytest.mark.parametrize("split", [True, False])
@pytest.mark.parametrize("dtype,D,H", [("f32", 16, 8), ("bf16", 32, 4)])
def test_heavy_groups_with_and_without_source_range_split(g, split, dtype, D, H):
    """Heavy rows on sorted rows with one head group, the plan's source-range
    groups in XCD order (xcd_split on) and the plain chunk groups (off): GT
    forward and backward, GATv2 forward and backward, each against the
    oracle."""
    import torch
    n = 3000
    say("heavy groups", "split" if split else "plain", dtype, D, H)
    ip, ix, rp, rx = _graph(g, 14, n)
    opts = dict(light_threshold=12, chunk=7, waves_per_group=4, want_csc=True)
    pl = g.gnn_plan_create(ip, ix, xcd_split=split, **opts)
    d = g.gnn_plan_export(pl)
    assert d["n_groups"] > 0 and d["rows_sorted"] == 1
    assert (d["n_xsplit_groups"] > 0) == split
    rng = np.random.default_rng(31 + D)
    Q, K, V, dO = rand_feats(rng, n, H, D, dtype, k=4)
    q, k, v, go = (dev_feat(x, dtype) for x in (Q, K, V, dO))
    O, L = g.gnn_attn_fwd(pl, ip, ix, q, k, v)
    ref = oracle.gt_fwd(rp, rx, Q, K, V)
    _check("GT O", host(O), ref["O"], ref["SO"], dtype)
    _check("GT LSE", host(L), ref["LSE"], ref["SL"], "f32")
    dq, dk, dv = g.gnn_attn_bwd(pl, ip, ix, q, k, v, O, go, L)
    rb = oracle.gt_bwd(rp, rx, Q, K, V, dO)
    for nm, x in (("dQ", dq), ("dK", dk), ("dV", dv)):
        _check(f"GT {nm}", host(x), rb[nm], rb["S" + nm], dtype)
    att = (rng.standard_normal((H, D)) / np.sqrt(D)).astype(np.float32)
    a = torch.from_numpy(att).cuda()
    GO, GL = g.gatv2_attn_fwd(pl, ip, ix, q, k, a)
    rg = oracle.gatv2_fwd(rp, rx, Q, K, att, slope=0.2)
    _check("GATv2 O", host(GO), rg["O"], rg["SO"], dtype)
    gxd, gxs, _, gda = g.gatv2_attn_bwd(pl, ip, ix, q, k, a, go, GL)
    rgb = oracle.gatv2_bwd(rp, rx, Q, K, att, dO, slope=0.2)
    _check("GATv2 dXD", host(gxd), rgb["dXD"], rgb["SdXD"], dtype)
    _check("GATv2 dXS", host(gxs), rgb["dXS"], rgb["SdXS"], dtype)
    _check("GATv2 d_att", gda.cpu().numpy(), rgb["d_att"], rgb["Sd_att"], dtype)
