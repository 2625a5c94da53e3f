"""Seeded random configurations across the library's option space, each
checked against the oracle: multigraphs from 1 to 3,000 nodes with skewed
in- and out-degrees, hubs (heavy rows and sources), empty rows and repeated
entries; fp32 or bf16; H in {1, 2, 3, 4, 8}, D in {16, 32, 64, 128}; no plan,
or a plan with a random light threshold, chunk, waves per group, launch
order and tile density, and in some graphs 16x16 block pairs filled to
60-100 % (so tiled plans have tiles). Every case runs the GT forward, the GATv2 forward,
the max reduction and, with a plan, the GT and GATv2 backward, the
reduction's gradient and both SpMM products, with guard bands around every
output and a check that no input changed."""
import numpy as np
import pytest

import oracle
from _gpu import check, dev_feat, dev_i32, host, rand_feats, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def g():
    import io_aware_sparse_amd as g
    g.lib()
    return g


def _case(seed):
    rng = np.random.default_rng(5000 + seed)
    n = int(rng.choice([1, 17, 300, 1500, 3000]))
    deg = rng.poisson(rng.uniform(0.5, 30), n)
    if n > 20 and rng.random() < 0.7:
        hubs = rng.choice(n, int(rng.integers(1, 6)), replace=False)
        deg[hubs] = rng.integers(100, 2500, hubs.size)
    deg[rng.random(n) < 0.05] = 0
    popular = rng.choice(n, max(1, n // 50), replace=False)          # skewed out-degrees
    rows = []
    for d in deg:
        src = rng.integers(0, n, d)
        pick = rng.random(d) < 0.3
        src[pick] = popular[rng.integers(0, popular.size, int(pick.sum()))]
        rows.append(src)
    if n >= 32 and rng.random() < 0.6:
        # locally dense spots: 16x16 block pairs filled to 60-100 % (tiles)
        nb = n // 16
        for _ in range(int(rng.integers(1, 8))):
            rb, cb = rng.integers(0, nb, 2)
            fill = rng.random((16, 16)) < rng.uniform(0.6, 1.0)
            for a in range(16):
                rows[rb * 16 + a] = np.concatenate([rows[rb * 16 + a], cb * 16 + np.nonzero(fill[a])[0]])
    rows = [np.sort(r) for r in rows]
    deg = np.array([r.size for r in rows], np.int64)
    ip = np.concatenate([[0], np.cumsum(deg)]).astype(np.int32)
    ix = np.concatenate(rows + [np.zeros(0, np.int64)]).astype(np.int32)
    dtype = str(rng.choice(["f32", "bf16"]))
    D = int(rng.choice([16, 32, 64, 128]))
    H = int(rng.choice([1, 2, 3, 4, 8]))
    opts = None
    if rng.random() >= 0.15:
        opts = dict(light_threshold=int(rng.choice([0, 3, 16, 64, 512])), chunk=int(rng.choice([1, 7, 64, 512])),
                    waves_per_group=int(rng.choice([1, 2, 4, 8])), sched_order=int(rng.integers(0, 3)),
                    tile_density=float(rng.choice([0.0, 0.5, 0.75])), want_csc=True)
    return n, ip, ix, dtype, H, D, opts, rng


@pytest.mark.parametrize("seed", range(400))
def test_random_configuration(g, seed):
    import torch
    n, ip, ix, dtype, H, D, opts, rng = _case(seed)
    say(f"random {seed}: N={n} E={ix.size} max deg={np.diff(ip).max() if n else 0} {dtype} H={H} D={D} plan={opts}")
    ipd, ixd = dev_i32(ip), dev_i32(ix)
    plan = g.gnn_plan_create(ipd, ixd, **opts) if opts else None
    if plan is not None and opts["tile_density"] > 0:
        say(f"  tiles {g.gnn_plan_export(plan)['n_tiles']}")
    Q, K, V, dO = rand_feats(rng, n, H, D, dtype, k=4)
    q, k, v, go = (dev_feat(x, dtype) for x in (Q, K, V, dO))
    # Every output buffer starts as NaN (an element a kernel leaves unwritten
    # fails the comparison) and sits between two guard bands of 64 NaN
    # elements that must stay untouched (a write past either end of an output
    # shows up there); the inputs must be left as they were.
    guards, G = [], 64

    def guarded(shape, dt, fill):
        size = int(np.prod(shape))
        b = torch.full((size + 2 * G,), fill, dtype=dt, device="cuda")
        guards.append((b, size, fill))
        return b[G:G + size].view(shape)

    nan = lambda shape, dt=q.dtype: guarded(shape, dt, float("nan"))                    # noqa: E731
    feat, stat = (n, H, D), (n, H)
    inputs = {"indptr": ipd, "indices": ixd, "Q": q, "K": k, "V": v, "dO": go}
    before = {nm: t.clone() for nm, t in inputs.items()}
    # GT forward (and backward on a plan)
    O, L = g.gnn_attn_fwd(plan, ipd, ixd, q, k, v, O=nan(feat), LSE=nan(stat, torch.float32))
    ref = oracle.gt_fwd(ip, ix, Q, K, V)
    check("GT O", host(O), ref["O"], ref["SO"], dtype)
    check("GT LSE", host(L), ref["LSE"], ref["SL"], "f32")
    if plan is not None:
        dq, dk, dv = g.gnn_attn_bwd(plan, ipd, ixd, q, k, v, O, go, L, dQ=nan(feat), dK=nan(feat), dV=nan(feat))
        rb = oracle.gt_bwd(ip, ix, Q, K, V, dO)
        for nm, x in (("dQ", dq), ("dK", dk), ("dV", dv)):
            check(f"GT {nm}", host(x), rb[nm], rb["S" + nm], dtype)
    # GATv2 forward (and backward on a plan), values aliasing XS
    att = (rng.standard_normal((H, D)) / np.sqrt(D)).astype(np.float32)
    a = torch.from_numpy(att).cuda()
    GO, GL = g.gatv2_attn_fwd(plan, ipd, ixd, q, k, a, O=nan(feat), LSE=nan(stat, torch.float32))
    rg = oracle.gatv2_fwd(ip, ix, Q, K, att, slope=0.2)
    check("GATv2 O", host(GO), rg["O"], rg["SO"], dtype)
    if plan is not None:
        gxd, gxs, _, gda = g.gatv2_attn_bwd(plan, ipd, ixd, q, k, a, go, GL, dXD=nan(feat), dXS=nan(feat),
                                            d_att=nan((H, D), torch.float32))
        rgb = oracle.gatv2_bwd(ip, ix, Q, K, att, dO, slope=0.2)
        check("GATv2 dXD", host(gxd), rgb["dXD"], rgb["SdXD"], dtype)
        check("GATv2 dXS", host(gxs), rgb["dXS"], rgb["SdXS"], dtype)
        check("GATv2 d_att", gda.cpu().numpy(), rgb["d_att"], rgb["Sd_att"], dtype)
    # max reduction: values and winners bit for bit (and the gradient on a plan)
    F = H * D
    X = q.reshape(n, F)
    out, arg = g.gnn_reduce_fwd(plan, ipd, ixd, X, "max", "src", out=nan((n, F)),
                                arg=guarded((n, F), torch.int32, 12345))
    rr = oracle.segment_reduce(ip, ix, Q.reshape(n, F), "max", "src")
    torch.cuda.synchronize()
    assert np.array_equal(arg.cpu().numpy(), rr["arg"]), "winners differ"
    assert np.array_equal(out.float().cpu().numpy(), rr["out"]), "values differ"
    if plan is not None:
        dX = g.gnn_reduce_bwd(plan, ipd, ixd, go.reshape(n, F), arg, "src", dX=nan((n, F)))
        rdx, S = oracle.segment_reduce_bwd(ip, ix, dO.reshape(n, F), rr["arg"], "src", want_scale=True)
        check("max dX", host(dX), rdx, S, dtype)
        # SpMM, both products
        g.gnn_spmm_prepare(plan, "gcn")
        for tr in (False, True):
            Y = g.gnn_spmm(plan, ipd, ixd, X, transpose=tr, Y=nan((n, F)))
            rs = oracle.spmm(ip, ix, Q.reshape(n, F), "gcn", transpose=tr)
            check(f"SpMM transpose={tr}", host(Y), rs["Y"], rs["S"], dtype)
    torch.cuda.synchronize()
    for b, size, fill in guards:
        band = torch.cat([b[:G], b[G + size:]])
        ok = torch.isnan(band).all() if b.is_floating_point() else (band == fill).all()
        assert ok.item(), "a write landed outside an output"
    for nm, t in inputs.items():
        assert torch.equal(t, before[nm]), f"input {nm} was modified"
