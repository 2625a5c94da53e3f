"""Full-graph parity at the benchmark's launch configuration (default plan:
T = 512, C = 512, W = 4) on every attention workload, and with the 16x16
tile path (tau = 0.75) on the two clustered graphs.

The CSR, buckets, transposed adjacency and (tiled plans) the tile census are
compared bit for bit over the whole graph. Every output row of every
attention workload is compared with the oracle: O and LSE for all rows, dQ
for all destination rows, dK and dV for all sources. The oracle runs over
row ranges of a few million edges at a time (progress lines in between); the
GPU outputs of each plan are compared with the same oracle rows. Properties
that hold at any size are checked on the full GPU outputs.

The reduction and SpMM workloads (ranked after the attention path) are
compared on every row, the SpMM on the clustered graph also on its tiled
plan; the reduction's gradient on every source up to 10M edges and, on the
64M-edge graph, on sampled sources and through a column-sum identity."""
import time

import numpy as np
import pytest

import oracle
import workloads
from _gpu import TOL, check, say

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

FULL = ["gt_uniform_n2708", "gt_chunglu25_n169k", "gatv2_zipf21_n100k", "gt_chunglu22_n2450k",
        "gt_comm16_n1m_deg27", "gt_comm16_n1m_deg100"]
TILED = {"gt_comm16_n1m_deg27", "gt_comm16_n1m_deg100"}
CHUNK_EDGES = 6_000_000          # oracle edges per call
N_SAMPLE = 20000                 # sampled sources of the reduction gradient on the 64M-edge graph


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


def _host32(t):
    """Device tensor -> host fp32 numpy (bf16 widened exactly)."""
    import torch
    return t.float().cpu().numpy() if t.dtype == torch.bfloat16 else t.cpu().numpy()


def _host(t):
    return _host32(t).astype(np.float64)


def _sample(rng, n, heavy, k):
    if n <= k + heavy.size:
        return np.arange(n)
    return np.unique(np.concatenate([heavy.astype(np.int64), rng.choice(n, k, replace=False)]))


def _check(name, x, ref, scale, dtype):
    check(name, x, ref, scale, dtype, f" over {np.asarray(ref).shape[0]} rows")


def row_ranges(indptr, edges_per_range):
    """Consecutive row ranges [lo, hi) of about edges_per_range entries each
    (at least one row per range) covering every row."""
    ip = np.asarray(indptr, np.int64)
    n = ip.size - 1
    out, lo = [], 0
    while lo < n:
        hi = int(np.searchsorted(ip, ip[lo] + edges_per_range, side="right")) - 1
        hi = min(n, max(hi, lo + 1))
        out.append((lo, hi))
        lo = hi
    return out


class Tracker:
    """Largest condition-scaled error and the normwise error of each output
    over every compared chunk; asserts the tolerance per chunk."""

    def __init__(self):
        self.err, self.num, self.den, self.rows = {}, {}, {}, {}

    def add(self, key, x, ref, scale, tol):
        e = oracle.scaled_error(x, ref, scale)
        x = np.asarray(x, np.float64)
        ref = np.asarray(ref, np.float64)
        fin = np.isfinite(ref)
        num = float(np.max(np.abs(x[fin] - ref[fin]))) if fin.any() else 0.0
        den = float(np.max(np.abs(ref[fin]))) if fin.any() else 0.0
        self.err[key] = max(self.err.get(key, 0.0), e)
        self.num[key] = max(self.num.get(key, 0.0), num)
        self.den[key] = max(self.den.get(key, 0.0), den)
        self.rows[key] = self.rows.get(key, 0) + ref.shape[0]
        assert e <= tol, (key, e)

    def report(self, out):
        for key in sorted(self.err):
            nw = self.num[key] / self.den[key] if self.den[key] > 0 else 0.0
            out(f"  {key[0]:>5} {key[1]:>4}: scaled err {self.err[key]:.3e}, normwise {nw:.3e} "
                f"over all {self.rows[key]} rows")


def _bits_equal(name, got, want):
    assert np.array_equal(np.asarray(got), np.asarray(want)), name


@pytest.mark.parametrize("name", FULL)
def test_full_graph(g, live, name):
    import torch
    t_start = time.time()
    live(f"\n[full] {name}: generating")
    say("full-graph", name)
    wl = workloads.make(name)
    n, H, D = wl.n_nodes, wl.heads, wl.dim
    ip, ix = g.gnn_csr_build(torch.from_numpy(wl.src).cuda(), torch.from_numpy(wl.dst).cuda(), n)
    rp, rx = oracle.csr_build(wl.src, wl.dst, n)
    _bits_equal("indptr", ip.cpu().numpy(), rp)
    _bits_equal("indices", ix.cpu().numpy(), rx)
    E = rx.size
    live(f"[full] {name}: CSR bit-exact, N = {n}, E = {E} ({time.time() - t_start:.0f} s)")
    ref_b = oracle.bucketing(rp, 512, 512, 4)
    if wl.backward:
        cip, cix = oracle.csc(rp, rx, n)
        ref_c = oracle.bucketing(cip, 512, 512, 4)
    variants = ["csr"] + (["tiles"] if name in TILED else [])
    outs = {}
    for var in variants:
        tiled = var == "tiles"
        plan = g.gnn_plan_create(ip, ix, want_csc=wl.backward, tile_density=0.75 if tiled else 0.0)
        d = g.gnn_plan_export(plan, arrays=True)
        for k in ("light", "heavy", "groups", "partial_ofs"):
            _bits_equal(k, d[k], ref_b[k])
        _bits_equal("light_sched", d["light_sched"], oracle.launch_order(rp, ref_b["light"]))
        _bits_equal("light_by_degree", d["light_by_degree"], oracle.launch_order(rp, ref_b["light"], 3))
        if wl.backward:
            _bits_equal("cindptr", d["cindptr"], cip)
            _bits_equal("cindices", d["cindices"], cix)
            for k in ("light", "heavy", "groups", "partial_ofs"):
                _bits_equal("c_" + k, d["c_" + k], ref_c[k])
            _bits_equal("c_light_sched", d["c_light_sched"], oracle.launch_order(cip, ref_c["light"]))
        if tiled:
            rt = oracle.tile_census(rp, rx, n, d["tile_min_nnz"], 512)
            for k in ("tile_rc", "tile_mask", "tile_ptr", "trb", "rindptr", "rindices", "light_nt", "ctile",
                      "ctile_ptr", "tcb", "rcindptr", "rcindices", "c_light_nt"):
                _bits_equal(k, d[k], rt[k])
            assert d["n_tiles"] > 0
            live(f"[full] {name}: tile census bit-exact, {d['n_tiles']} tiles, "
                 f"{d['n_residual']} residual edges")
        live(f"[full] {name} [{var}]: plan bit-exact (light {d['n_light']}, heavy {d['n_heavy']}, "
             f"groups {d['n_groups']})")
        o = {}
        if wl.kind == "gatv2":
            xd, xs = _dev(wl, "XD"), _dev(wl, "XS")
            att = torch.from_numpy(wl.att).cuda()
            O, L = g.gatv2_attn_fwd(plan, ip, ix, xd, xs, att, negative_slope=0.2)
            torch.cuda.synchronize()
            o["O"], o["LSE"] = _host32(O), _host32(L)
            del xd, xs, O, L
        else:
            q, k, v = _dev(wl, "Q"), _dev(wl, "K"), _dev(wl, "V")
            O, L = g.gnn_attn_fwd(plan, ip, ix, q, k, v)
            torch.cuda.synchronize()
            o["O"], o["LSE"] = _host32(O), _host32(L)
            if not tiled:
                # the weights sum to one at any size
                Oc, _ = g.gnn_attn_fwd(plan, ip, ix, q, k, torch.full_like(v, 0.5), want_lse=False)
                assert torch.max(torch.abs(Oc.float() - 0.5)).item() <= (1e-5 if wl.dtype == "f32" else 4e-3)
                del Oc
            if wl.backward:
                go = _dev(wl, "dO")
                dq, dk, dv = g.gnn_attn_bwd(plan, ip, ix, q, k, v, O, go, L)
                torch.cuda.synchronize()
                # gradient identities on the full GPU outputs: sum_j dK_j = 0, sum_j dV_j = sum_i dO_i
                sdk = dk.double().sum(0).abs()
                sdv = (dv.double().sum(0) - go.double().sum(0)).abs()
                live(f"[full] {name} [{var}]: |sum dK| max {sdk.max().item():.3e}, "
                     f"|sum dV - sum dO| max {sdv.max().item():.3e}")
                assert torch.all(sdk <= 2e-2 * dk.double().abs().sum(0) + 1e-3)
                assert torch.all(sdv <= 2e-2 * dv.double().abs().sum(0) + 1e-3)
                o["dQ"], o["dK"], o["dV"] = _host32(dq), _host32(dk), _host32(dv)
                del go, dq, dk, dv
            del q, k, v, O, L
        outs[var] = o
        g.gnn_plan_destroy(plan)
        torch.cuda.empty_cache()
        live(f"[full] {name} [{var}]: GPU outputs on the host ({time.time() - t_start:.0f} s)")

    # the oracle over every row, a range of rows at a time
    tol = TOL[wl.dtype]
    tr = Tracker()
    f64 = {k: np.asarray(v, np.float64) for k, v in wl.feats.items()}
    if wl.backward:
        M = np.empty((n, H)); Z = np.empty((n, H)); Dl = np.empty((n, H))
    ranges = row_ranges(rp, CHUNK_EDGES)
    t0 = time.time()
    for c, (lo, hi) in enumerate(ranges):
        rows = np.arange(lo, hi)
        if wl.kind == "gatv2":
            ref = oracle.gatv2_fwd(rp, rx, f64["XD"], f64["XS"], wl.att, slope=0.2, rows=rows)
        else:
            ref = oracle.gt_fwd(rp, rx, f64["Q"], f64["K"], f64["V"], rows=rows)
        for var in variants:
            tr.add((var, "O"), outs[var]["O"][lo:hi], ref["O"], ref["SO"], tol)
            tr.add((var, "LSE"), outs[var]["LSE"][lo:hi], ref["LSE"], ref["SL"], TOL["f32"])
        if wl.backward:
            rb = oracle.gt_bwd_dst(rp, rx, f64["Q"], f64["K"], f64["V"], f64["dO"], rows=rows)
            M[lo:hi], Z[lo:hi], Dl[lo:hi] = rb["M"], rb["Z"], rb["Delta"]
            for var in variants:
                tr.add((var, "dQ"), outs[var]["dQ"][lo:hi], rb["dQ"], rb["SdQ"], tol)
        if len(ranges) > 1:
            live(f"[full] {name}: rows {hi}/{n} compared ({time.time() - t0:.0f} s)")
    if wl.backward:
        cranges = row_ranges(cip, CHUNK_EDGES)
        for lo, hi in cranges:
            rs = oracle.gt_bwd_src(cip, cix, f64["Q"], f64["K"], f64["V"], f64["dO"], M, Z, Dl,
                                   srcs=np.arange(lo, hi))
            for var in variants:
                tr.add((var, "dK"), outs[var]["dK"][lo:hi], rs["dK"], rs["SdK"], tol)
                tr.add((var, "dV"), outs[var]["dV"][lo:hi], rs["dV"], rs["SdV"], tol)
            live(f"[full] {name}: sources {hi}/{n} compared ({time.time() - t0:.0f} s)")
    live(f"[full] {name}: every row compared (tol {tol:.0e}; LSE 1e-4), {time.time() - t_start:.0f} s in all")
    tr.report(live)
    assert tr.rows[("csr", "O")] == n


def test_full_graph_gatv2_backward(g, live):
    """GATv2 forward + backward on the Zipf(2.1) graph (N = 100,000,
    E = 5.1M, H = 8, D = 16, fp32) with a seeded upstream gradient: dXD on
    every row, dXS on every source, d_att over every edge."""
    import torch
    name = "gatv2_zipf21_n100k"
    say("full-graph backward", name)
    t0 = time.time()
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
    ref = oracle.gatv2_bwd(rp, rx, wl.feats["XD"], wl.feats["XS"], wl.att, wl.feats["dO"], slope=0.2,
                           csc_arrays=(cip, cix))
    _check("dXD", _host(gxd), ref["dXD"], ref["SdXD"], "f32")
    _check("dXS", _host(gxs), ref["dXS"], ref["SdXS"], "f32")
    _check("d_att", gda.cpu().numpy(), ref["d_att"], ref["Sd_att"], "f32")
    live(f"[full] {name} backward: every row and source compared ({time.time() - t0:.0f} s)")


def _bits32(x):
    return np.ascontiguousarray(x, np.float32).view(np.uint32)


@pytest.mark.parametrize("name", ["maxpool_zipf21_n100k", "maxpool_chunglu22_n2450k"])
def test_full_size_reduce(g, live, name):
    """Max / min reduction at full size, default plan: values and winners bit
    for bit on every row; the gradient against the oracle on every source
    (Zipf graph) or, on the 64M-edge graph, on every heavy source and a
    seeded sample of light ones (max of sources: the oracle given only the
    winners that fall in the sample, so that its scatter stays small) and
    through its column-sum identity (every non-empty row's dOut lands exactly
    once)."""
    import torch
    say("full-size reduce", name)
    t0 = time.time()
    wl = workloads.make(name, backward=True)
    n, F = wl.n_nodes, wl.heads * wl.dim
    ip, ix = g.gnn_csr_build(torch.from_numpy(wl.src).cuda(), torch.from_numpy(wl.dst).cuda(), n)
    rp, rx = oracle.csr_build(wl.src, wl.dst, n)
    assert np.array_equal(ip.cpu().numpy(), rp) and np.array_equal(ix.cpu().numpy(), rx)
    small = rx.size <= 10_000_000
    plan = g.gnn_plan_create(ip, ix, want_csc=True)
    heavy = oracle.bucketing(rp, 512, 512, 4)["heavy"]
    cip, _ = oracle.csc(rp, rx, n)
    rng = np.random.default_rng(79)
    rows = np.arange(n)
    srcs = None if small else _sample(rng, n, oracle.bucketing(cip, 512, 512, 4)["heavy"], N_SAMPLE)
    X = wl.feats["X"].reshape(n, F)
    Xd = _dev(wl, "X").reshape(n, F)
    gO = _dev(wl, "dO").reshape(n, F)
    for op, msg in (("max", "src"), ("min", "diff")):
        out, arg = g.gnn_reduce_fwd(plan, ip, ix, Xd, op, msg)
        torch.cuda.synchronize()
        ref = oracle.segment_reduce(rp, rx, X, op, msg)
        ro = oracle.round_bf16(ref["out"]) if (wl.dtype == "bf16" and msg == "diff") else ref["out"]
        ga = arg.cpu().numpy()[rows]
        go = out.float().cpu().numpy()[rows]
        say(f"  {op} {msg}: every row ({heavy.size} heavy), winners equal "
            f"{np.mean(ga == ref['arg']):.6f}, values equal {np.mean(_bits32(go) == _bits32(ro)):.6f}")
        assert np.array_equal(ga, ref["arg"]) and np.array_equal(_bits32(go), _bits32(ro)), (op, msg)
        dX = g.gnn_reduce_bwd(plan, ip, ix, gO, arg, msg)
        torch.cuda.synchronize()
        if small:
            rdX, S = oracle.segment_reduce_bwd(rp, rx, wl.feats["dO"].reshape(n, F), ref["arg"], msg,
                                               want_scale=True)
            _check(f"dX {op} {msg}", _host(dX), rdX, S, wl.dtype)
        else:
            if msg == "src":
                # every term that lands on a sampled source: the winners outside the sample dropped
                keep = np.where(np.isin(ref["arg"], srcs), ref["arg"], -1)
                rdX, S = oracle.segment_reduce_bwd(rp, rx, wl.feats["dO"].reshape(n, F), keep, msg,
                                                   want_scale=True)
                _check(f"dX {op} {msg} (sampled sources)", _host(dX)[srcs], rdX[srcs], S[srcs], wl.dtype)
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
    live(f"[full] {name}: every row compared{'' if small else f', {srcs.size} sources of the gradient'} "
         f"({time.time() - t0:.0f} s)")


@pytest.mark.parametrize("name,tau", [("spmm_chunglu25_n169k", 0.0), ("spmm_chunglu22_n2450k", 0.0),
                                      ("spmm_comm16_n1m_deg27", 0.0), ("spmm_comm16_n1m_deg27", 0.75)])
def test_full_size_spmm(g, live, name, tau):
    """GCN-normalised SpMM and its transpose at full size, on the default plan
    and (clustered graph) on the tiled plan the benchmark times, whose tiled
    blocks run on the 16x16 block kernel: every row and every source."""
    import torch
    say("full-size spmm", name, "tile density", tau)
    t0 = time.time()
    wl = workloads.make(name, backward=True)
    n, F = wl.n_nodes, wl.heads * wl.dim
    ip, ix = g.gnn_csr_build(torch.from_numpy(wl.src).cuda(), torch.from_numpy(wl.dst).cuda(), n)
    rp, rx = oracle.csr_build(wl.src, wl.dst, n)
    assert np.array_equal(ip.cpu().numpy(), rp) and np.array_equal(ix.cpu().numpy(), rx)
    plan = g.gnn_plan_create(ip, ix, want_csc=True, tile_density=tau)
    if tau > 0:
        info = g.gnn_plan_export(plan)
        say(f"  tiles {info['n_tiles']}, tiled row blocks {info['n_trb']}, column blocks {info['n_tcb']}")
        assert info["n_trb"] > 0 and info["n_tcb"] > 0
    g.gnn_spmm_prepare(plan, "gcn")
    rows = srcs = np.arange(n)
    X = wl.feats["X"].reshape(n, F)
    dO = wl.feats["dO"].reshape(n, F)
    Y = g.gnn_spmm(plan, ip, ix, _dev(wl, "X").reshape(n, F))
    dX = g.gnn_spmm(plan, ip, ix, _dev(wl, "dO").reshape(n, F), transpose=True)
    torch.cuda.synchronize()
    ref = oracle.spmm(rp, rx, X, "gcn", rows=rows)
    _check("Y", _host(Y)[rows], ref["Y"], ref["S"], wl.dtype)
    ref = oracle.spmm(rp, rx, dO, "gcn", transpose=True, rows=srcs)
    _check("dX", _host(dX)[srcs], ref["Y"], ref["S"], wl.dtype)
    live(f"[full] {name}: every row and source compared ({time.time() - t0:.0f} s)")
