"""Full-size parity at the benchmark's launch configuration (default plan:
T = 512, C = 512, W = 4) on every workload.

The CSR, buckets and transposed adjacency are compared bit for bit over the
whole graph. Outputs are compared on sampled rows the oracle computes one by
one: every heavy row (heavy sources for dK/dV) plus seeded uniform samples
of light rows; the small workloads are compared in full. Properties that
hold at any size are checked on the full GPU outputs."""
import numpy as np
import pytest

import oracle
import workloads
from _gpu import TOL, say

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

FULL = ["gt_uniform_n2708", "gt_chunglu25_n169k", "gatv2_zipf21_n100k", "gt_chunglu22_n2450k",
        "gt_comm16_n1m_deg100", "gt_comm16_n1m_deg27"]
N_SAMPLE = 20000


@pytest.fixture(scope="module")
def g():
    import io_aware_sparse_amd as g
    g.lib()
    return g


def _dev(wl, nm):
    import torch
    if wl.dtype == "bf16":
        return torch.from_numpy(wl.bits[nm].view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(wl.feats[nm]).cuda()


def _host(t):
    import torch
    return t.float().cpu().numpy().astype(np.float64) if t.dtype == torch.bfloat16 else t.cpu().numpy().astype(np.float64)


def _sample(rng, n, heavy, k):
    if n <= k + heavy.size:
        return np.arange(n)
    return np.unique(np.concatenate([heavy.astype(np.int64), rng.choice(n, k, replace=False)]))


def _check(name, x, ref, scale, dtype):
    err = oracle.scaled_error(x, ref, scale)
    say(f"  {name}: scaled err {err:.3e} over {np.asarray(ref).shape[0]} rows (tol {TOL[dtype]:.0e})")
    assert err <= TOL[dtype], (name, err)


@pytest.mark.parametrize("name", FULL)
def test_full_size(g, name):
    import torch
    say("full-size", name)
    wl = workloads.make(name)
    n, H, D = wl.n_nodes, wl.heads, wl.dim
    ip, ix = g.gnn_csr_build(torch.from_numpy(wl.src).cuda(), torch.from_numpy(wl.dst).cuda(), n)
    rp, rx = oracle.csr_build(wl.src, wl.dst, n)
    assert np.array_equal(ip.cpu().numpy(), rp), "indptr"
    assert np.array_equal(ix.cpu().numpy(), rx), "indices"
    say("  CSR bit-exact, E =", rx.size)
    plan = g.gnn_plan_create(ip, ix, want_csc=wl.backward)
    d = g.gnn_plan_export(plan, arrays=True)
    ref_b = oracle.bucketing(rp, 512, 512, 4)
    for k in ("light", "heavy", "groups", "partial_ofs"):
        assert np.array_equal(d[k], ref_b[k]), k
    assert np.array_equal(d["light_sched"], oracle.launch_order(rp, ref_b["light"])), "light_sched"
    assert np.array_equal(d["light_by_degree"], oracle.launch_order(rp, ref_b["light"], 1)), "light_by_degree"
    if wl.backward:
        cip, cix = oracle.csc(rp, rx, n)
        assert np.array_equal(d["cindptr"], cip) and np.array_equal(d["cindices"], cix), "csc"
        ref_c = oracle.bucketing(cip, 512, 512, 4)
        for k in ("light", "heavy", "groups", "partial_ofs"):
            assert np.array_equal(d["c_" + k], ref_c[k]), "c_" + k
        assert np.array_equal(d["c_light_sched"], oracle.launch_order(cip, ref_c["light"])), "c_light_sched"
    say(f"  buckets bit-exact: light {d['n_light']} heavy {d['n_heavy']} groups {d['n_groups']}")
    rng = np.random.default_rng(77)
    rows = _sample(rng, n, ref_b["heavy"], N_SAMPLE)
    if wl.kind == "gatv2":
        xd, xs = _dev(wl, "XD"), _dev(wl, "XS")
        att = torch.from_numpy(wl.att).cuda()
        O, L = g.gatv2_attn_fwd(plan, ip, ix, xd, xs, att, negative_slope=0.2)
        torch.cuda.synchronize()
        ref = oracle.gatv2_fwd(rp, rx, wl.feats["XD"], wl.feats["XS"], wl.att, slope=0.2, rows=rows)
        _check("O", _host(O)[rows], ref["O"], ref["SO"], wl.dtype)
        _check("LSE", _host(L)[rows], ref["LSE"], ref["SL"], "f32")
        return
    q, k, v = _dev(wl, "Q"), _dev(wl, "K"), _dev(wl, "V")
    O, L = g.gnn_attn_fwd(plan, ip, ix, q, k, v)
    torch.cuda.synchronize()
    Q = np.asarray(wl.feats["Q"], np.float64)
    K = np.asarray(wl.feats["K"], np.float64)
    V = np.asarray(wl.feats["V"], np.float64)
    ref = oracle.gt_fwd(rp, rx, Q, K, V, rows=rows)
    _check("O", _host(O)[rows], ref["O"], ref["SO"], wl.dtype)
    _check("LSE", _host(L)[rows], ref["LSE"], ref["SL"], "f32")
    # weights sum to one at any size
    Oc, _ = g.gnn_attn_fwd(plan, ip, ix, q, k, torch.full_like(v, 0.5), want_lse=False)
    assert torch.max(torch.abs(Oc.float() - 0.5)).item() <= (1e-5 if wl.dtype == "f32" else 4e-3)
    del Oc
    if not wl.backward:
        return
    go = _dev(wl, "dO")
    dq, dk, dv = g.gnn_attn_bwd(plan, ip, ix, q, k, v, O, go, L)
    torch.cuda.synchronize()
    srcs = _sample(rng, n, ref_c["heavy"], N_SAMPLE // 4)
    dO = np.asarray(wl.feats["dO"], np.float64)
    rb = oracle.gt_bwd(rp, rx, Q, K, V, dO, rows=rows, srcs=srcs, csc_arrays=(cip, cix))
    _check("dQ", _host(dq)[rows], rb["dQ"], rb["SdQ"], wl.dtype)
    _check("dK", _host(dk)[srcs], rb["dK"], rb["SdK"], wl.dtype)
    _check("dV", _host(dv)[srcs], rb["dV"], rb["SdV"], wl.dtype)
    # gradient identities on the full GPU outputs
    sdk = dk.double().sum(0).abs()
    sdv = (dv.double().sum(0) - go.double().sum(0)).abs()
    say(f"  |sum dK| max {sdk.max().item():.3e}, |sum dV - sum dO| max {sdv.max().item():.3e}")
    assert torch.all(sdk <= 2e-2 * dk.double().abs().sum(0) + 1e-3)
    assert torch.all(sdv <= 2e-2 * dv.double().abs().sum(0) + 1e-3)


def test_full_size_gatv2_backward(g):
    """GATv2 forward + backward on the Zipf(2.1) graph (N = 100,000,
    E = 5.1M, H = 8, D = 16, fp32) with a seeded upstream gradient."""
    import torch
    name = "gatv2_zipf21_n100k"
    say("full-size backward", name)
    wl = workloads.make(name, backward=True)
    n = wl.n_nodes
    ip, ix = g.gnn_csr_build(torch.from_numpy(wl.src).cuda(), torch.from_numpy(wl.dst).cuda(), n)
    rp, rx = oracle.csr_build(wl.src, wl.dst, n)
    assert np.array_equal(ip.cpu().numpy(), rp) and np.array_equal(ix.cpu().numpy(), rx)
    plan = g.gnn_plan_create(ip, ix, want_csc=True)
    cip, cix = oracle.csc(rp, rx, n)
    xd, xs, go = _dev(wl, "XD"), _dev(wl, "XS"), _dev(wl, "dO")
    att = torch.from_numpy(wl.att).cuda()
    O, L = g.gatv2_attn_fwd(plan, ip, ix, xd, xs, att)
    gxd, gxs, _, gda = g.gatv2_attn_bwd(plan, ip, ix, xd, xs, att, go, L)
    torch.cuda.synchronize()
    rng = np.random.default_rng(78)
    rows = _sample(rng, n, oracle.bucketing(rp, 512, 512, 4)["heavy"], N_SAMPLE)
    srcs = _sample(rng, n, oracle.bucketing(cip, 512, 512, 4)["heavy"], N_SAMPLE // 4)
    ref = oracle.gatv2_bwd(rp, rx, wl.feats["XD"], wl.feats["XS"], wl.att, wl.feats["dO"], slope=0.2, rows=rows,
                           srcs=srcs, csc_arrays=(cip, cix))
    _check("dXD", _host(gxd)[rows], ref["dXD"], ref["SdXD"], "f32")
    _check("dXS", _host(gxs)[srcs], ref["dXS"], ref["SdXS"], "f32")
    _check("d_att", gda.cpu().numpy(), ref["d_att"], ref["Sd_att"], "f32")


def _bits32(x):
    return np.ascontiguousarray(x, np.float32).view(np.uint32)


@pytest.mark.parametrize("name", ["maxpool_zipf21_n100k", "maxpool_chunglu22_n2450k"])
def test_full_size_reduce(g, name):
    """Max / min reduction at full size, default plan: values and winners bit
    for bit on every heavy row and a seeded sample of light rows; the
    gradient against the oracle on sampled sources (Zipf graph) or through
    its column-sum identity (every non-empty row's dOut lands exactly once)."""
    import torch
    say("full-size reduce", name)
    wl = workloads.make(name, backward=True)
    n, F = wl.n_nodes, wl.heads * wl.dim
    ip, ix = g.gnn_csr_build(torch.from_numpy(wl.src).cuda(), torch.from_numpy(wl.dst).cuda(), n)
    rp, rx = oracle.csr_build(wl.src, wl.dst, n)
    assert np.array_equal(ip.cpu().numpy(), rp) and np.array_equal(ix.cpu().numpy(), rx)
    plan = g.gnn_plan_create(ip, ix, want_csc=True)
    heavy = oracle.bucketing(rp, 512, 512, 4)["heavy"]
    rng = np.random.default_rng(79)
    rows = _sample(rng, n, heavy, N_SAMPLE)
    X = wl.feats["X"].reshape(n, F)
    Xd = _dev(wl, "X").reshape(n, F)
    gO = _dev(wl, "dO").reshape(n, F)
    for op, msg in (("max", "src"), ("min", "diff")):
        out, arg = g.gnn_reduce_fwd(plan, ip, ix, Xd, op, msg)
        torch.cuda.synchronize()
        ref = oracle.segment_reduce(rp, rx, X, op, msg, rows=rows)
        ro = oracle.round_bf16(ref["out"]) if (wl.dtype == "bf16" and msg == "diff") else ref["out"]
        ga = arg.cpu().numpy()[rows]
        go = out.float().cpu().numpy()[rows]
        say(f"  {op} {msg}: {rows.size} rows ({heavy.size} heavy), winners equal "
            f"{np.mean(ga == ref['arg']):.6f}, values equal {np.mean(_bits32(go) == _bits32(ro)):.6f}")
        assert np.array_equal(ga, ref["arg"]) and np.array_equal(_bits32(go), _bits32(ro)), (op, msg)
        dX = g.gnn_reduce_bwd(plan, ip, ix, gO, arg, msg)
        torch.cuda.synchronize()
        if wl.n_nodes <= 200_000:
            full = oracle.segment_reduce(rp, rx, X, op, msg)["arg"]
            rdX, S = oracle.segment_reduce_bwd(rp, rx, wl.feats["dO"].reshape(n, F), full, msg, want_scale=True)
            cip, _ = oracle.csc(rp, rx, n)
            srcs = _sample(rng, n, oracle.bucketing(cip, 512, 512, 4)["heavy"], N_SAMPLE)
            _check(f"dX {op} {msg}", _host(dX)[srcs], rdX[srcs], S[srcs], wl.dtype)
        else:
            nonempty = np.diff(rp) > 0
            col = dX.double().sum(0).cpu().numpy()
            want = wl.feats["dO"].reshape(n, F)[nonempty].astype(np.float64).sum(0)
            if msg == "diff":
                want = want - want                   # each row's dOut comes in once and goes out once
            mag = np.abs(wl.feats["dO"].reshape(n, F)).astype(np.float64).sum(0)
            err = np.max(np.abs(col - want) / mag)
            say(f"  dX column sums: max |sum - expected| / sum|dOut| = {err:.2e}")
            assert err <= (1e-6 if wl.dtype == "f32" else 1e-2), err
        del out, arg, dX


@pytest.mark.parametrize("name", ["spmm_chunglu25_n169k", "spmm_chunglu22_n2450k"])
def test_full_size_spmm(g, name):
    """GCN-normalised SpMM and its transpose at full size, default plan, on
    every heavy row (source) and a seeded sample of light ones."""
    import torch
    say("full-size spmm", name)
    wl = workloads.make(name, backward=True)
    n, F = wl.n_nodes, wl.heads * wl.dim
    ip, ix = g.gnn_csr_build(torch.from_numpy(wl.src).cuda(), torch.from_numpy(wl.dst).cuda(), n)
    rp, rx = oracle.csr_build(wl.src, wl.dst, n)
    assert np.array_equal(ip.cpu().numpy(), rp) and np.array_equal(ix.cpu().numpy(), rx)
    plan = g.gnn_plan_create(ip, ix, want_csc=True)
    g.gnn_spmm_prepare(plan, "gcn")
    rng = np.random.default_rng(80)
    rows = _sample(rng, n, oracle.bucketing(rp, 512, 512, 4)["heavy"], N_SAMPLE)
    cip, _ = oracle.csc(rp, rx, n)
    srcs = _sample(rng, n, oracle.bucketing(cip, 512, 512, 4)["heavy"], N_SAMPLE)
    X = wl.feats["X"].reshape(n, F)
    dO = wl.feats["dO"].reshape(n, F)
    Y = g.gnn_spmm(plan, ip, ix, _dev(wl, "X").reshape(n, F))
    dX = g.gnn_spmm(plan, ip, ix, _dev(wl, "dO").reshape(n, F), transpose=True)
    torch.cuda.synchronize()
    ref = oracle.spmm(rp, rx, X, "gcn", rows=rows)
    _check("Y", _host(Y)[rows], ref["Y"], ref["S"], wl.dtype)
    ref = oracle.spmm(rp, rx, dO, "gcn", transpose=True, rows=srcs)
    _check("dX", _host(dX)[srcs], ref["Y"], ref["S"], wl.dtype)
