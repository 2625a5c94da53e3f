"""GPU parity of the degree-aware max / min reduction (gnn_reduce_fwd /
gnn_reduce_bwd) against the oracle.

The forward is exact, so values (signed zeros included) and winning sources
are compared bit for bit: fp32 and bf16, max and min, source and difference
messages, rows from one 16-byte slice to several waves wide, no plan, a plan
whose tiny threshold sends most rows through the chunked heavy path and its
64-bit atomics, and the default plan. Inputs are drawn from a few levels
(with -0 and +0) so that ties, which the smallest source must win, are
everywhere; graphs have empty rows and repeated sources. The backward is an
fp32 sum compared at the condition-scaled bar."""
import numpy as np
import pytest

import oracle
from _gpu import TOL, check, dev_feat, dev_i32, host, say

pytestmark = pytest.mark.gpu

LEVELS = np.array([-2.0, -0.5, -0.0, 0.0, 0.25, 1.0, 3.0], np.float32)


@pytest.fixture(scope="module")
def g():
    import io_aware_sparse_amd as g
    g.lib()
    return g


def _graph(rng, n, mean_deg, hub_deg=0, dup=0.05, empty=0.05):
    """CSR by destination with ascending sources, some repeated, some rows empty."""
    deg = rng.poisson(mean_deg, n)
    if hub_deg:
        deg[rng.choice(n, 3, replace=False)] = hub_deg
    deg[rng.random(n) < empty] = 0
    rows = []
    for i in range(n):
        s = rng.integers(0, n, deg[i])
        k = rng.random(deg[i]) < dup
        s = np.concatenate([s, s[k]])
        rows.append(np.sort(s))
    indptr = np.concatenate([[0], np.cumsum([r.size for r in rows])]).astype(np.int32)
    indices = np.concatenate(rows).astype(np.int32) if indptr[-1] else np.zeros(0, np.int32)
    return indptr, indices


def _feats(rng, n, F, dtype, ties=True):
    if ties:
        return rng.choice(LEVELS, (n, F))
    x = rng.standard_normal((n, F)).astype(np.float32)
    return oracle.round_bf16(x) if dtype == "bf16" else x


def _bits(x):
    return np.ascontiguousarray(x, np.float32).view(np.uint32)


def _gpu_out_f32(t):
    import torch
    return t.float().cpu().numpy() if t.dtype == torch.bfloat16 else t.cpu().numpy()


def _ref(ip, ix, X, op, msg, dtype, rows=None):
    r = oracle.segment_reduce(ip, ix, X, op, msg, rows=rows)
    out = r["out"]
    if dtype == "bf16" and msg == "diff":
        out = oracle.round_bf16(out)
    return out, r["arg"]


def _plan(g, ip_d, ix_d, kind, csc=False):
    if kind == "none":
        return None
    if kind == "tiny":
        return g.gnn_plan_create(ip_d, ix_d, light_threshold=3, chunk=2, waves_per_group=2, want_csc=csc)
    return g.gnn_plan_create(ip_d, ix_d, want_csc=csc)


CASES = [("f32", 4), ("f32", 32), ("f32", 96), ("f32", 128), ("f32", 256), ("f32", 320), ("bf16", 8), ("bf16", 64),
         ("bf16", 128), ("bf16", 200), ("bf16", 1032)]


@pytest.mark.parametrize("dtype,F", CASES)
@pytest.mark.parametrize("plan_kind", ["none", "tiny", "default"])
def test_reduce_fwd_exact(g, dtype, F, plan_kind):
    rng = np.random.default_rng(F * 7 + len(plan_kind))
    n = 700
    ip, ix = _graph(rng, n, 9, hub_deg=1500)
    X = _feats(rng, n, F, dtype)
    ip_d, ix_d = dev_i32(ip), dev_i32(ix)
    Xd = dev_feat(X, dtype)
    plan = _plan(g, ip_d, ix_d, plan_kind)
    if plan is not None:
        d = g.gnn_plan_export(plan)
        say(f"reduce fwd {dtype} F={F} plan={plan_kind}: light {d['n_light']} heavy {d['n_heavy']} "
            f"groups {d['n_groups']}")
    else:
        say(f"reduce fwd {dtype} F={F} plan=none")
    for op in ("max", "min"):
        for msg in ("src", "diff"):
            out, arg = g.gnn_reduce_fwd(plan, ip_d, ix_d, Xd, op, msg)
            ro, ra = _ref(ip, ix, X, op, msg, dtype)
            ga = arg.cpu().numpy()
            assert np.array_equal(ga, ra), (op, msg, np.argwhere(ga != ra)[:5])
            assert np.array_equal(_bits(_gpu_out_f32(out)), _bits(ro)), (op, msg)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_reduce_fwd_continuous_and_no_arg(g, dtype):
    """Continuous inputs (no ties) on a skewed graph; arg may be omitted."""
    rng = np.random.default_rng(9)
    n, F = 3000, 64
    ip, ix = _graph(rng, n, 20, hub_deg=5000, empty=0.01)
    X = _feats(rng, n, F, dtype, ties=False)
    ip_d, ix_d = dev_i32(ip), dev_i32(ix)
    plan = g.gnn_plan_create(ip_d, ix_d, light_threshold=64, chunk=32, waves_per_group=4)
    Xd = dev_feat(X, dtype)
    for op in ("max", "min"):
        out, arg = g.gnn_reduce_fwd(plan, ip_d, ix_d, Xd, op, "src")
        out2, none = g.gnn_reduce_fwd(plan, ip_d, ix_d, Xd, op, "src", want_arg=False)
        assert none is None
        ro, ra = _ref(ip, ix, X, op, "src", dtype)
        assert np.array_equal(arg.cpu().numpy(), ra)
        assert np.array_equal(_bits(_gpu_out_f32(out)), _bits(ro))
        assert np.array_equal(_bits(_gpu_out_f32(out2)), _bits(ro))


def test_reduce_fwd_edge_cases(g):
    import torch
    # all rows empty
    n, F = 50, 8
    ip = np.zeros(n + 1, np.int32)
    ix = np.zeros(0, np.int32)
    X = np.ones((n, F), np.float32)
    out, arg = g.gnn_reduce_fwd(None, dev_i32(ip), dev_i32(ix), dev_feat(X, "f32"), "max", "diff")
    assert torch.all(out == 0).item() and torch.all(arg == -1).item()
    # empty graph
    out, arg = g.gnn_reduce_fwd(None, dev_i32(np.zeros(1, np.int32)), dev_i32(ix),
                                dev_feat(np.zeros((0, F), np.float32), "f32"), "min")
    assert out.numel() == 0
    # one row holding every node, including itself many times
    n = 300
    ix = np.sort(np.concatenate([np.arange(n), np.full(50, 7)])).astype(np.int32)
    ip = np.zeros(n + 1, np.int32)
    ip[1:] = ix.size
    rng = np.random.default_rng(5)
    X = _feats(rng, n, 16, "f32")
    ip_d, ix_d = dev_i32(ip), dev_i32(ix)
    for plan in (None, g.gnn_plan_create(ip_d, ix_d, light_threshold=10, chunk=7, waves_per_group=8)):
        for op in ("max", "min"):
            out, arg = g.gnn_reduce_fwd(plan, ip_d, ix_d, dev_feat(X, "f32"), op, "diff")
            ro, ra = _ref(ip, ix, X, op, "diff", "f32")
            assert np.array_equal(arg.cpu().numpy(), ra) and np.array_equal(_bits(out.cpu().numpy()), _bits(ro))


@pytest.mark.parametrize("dtype,F", [("f32", 4), ("f32", 128), ("f32", 320), ("bf16", 8), ("bf16", 128),
                                     ("bf16", 1032)])
@pytest.mark.parametrize("plan_kind", ["tiny", "default"])
def test_reduce_bwd(g, dtype, F, plan_kind):
    rng = np.random.default_rng(F + 100)
    n = 600
    ip, ix = _graph(rng, n, 8, hub_deg=900)
    X = _feats(rng, n, F, dtype)
    dOut = _feats(rng, n, F, dtype, ties=False)
    ip_d, ix_d = dev_i32(ip), dev_i32(ix)
    plan = _plan(g, ip_d, ix_d, plan_kind, csc=True)
    d = g.gnn_plan_export(plan)
    say(f"reduce bwd {dtype} F={F} plan={plan_kind}: sources light {d['c_n_light']} heavy {d['c_n_heavy']}")
    Xd, gd = dev_feat(X, dtype), dev_feat(dOut, dtype)
    for op in ("max", "min"):
        for msg in ("src", "diff"):
            _, arg = g.gnn_reduce_fwd(plan, ip_d, ix_d, Xd, op, msg)
            dX = g.gnn_reduce_bwd(plan, ip_d, ix_d, gd, arg, msg)
            ra = oracle.segment_reduce(ip, ix, X, op, msg)["arg"]
            ref, S = oracle.segment_reduce_bwd(ip, ix, dOut, ra, msg, want_scale=True)
            check(f"{op} {msg} dX", host(dX), ref, S, dtype)
            dX2 = g.gnn_reduce_bwd(plan, ip_d, ix_d, gd, arg, msg)
            assert np.array_equal(host(dX2), host(dX)), "not reproducible"


def test_reduce_bwd_needs_csc(g):
    rng = np.random.default_rng(1)
    ip, ix = _graph(rng, 40, 3)
    ip_d, ix_d = dev_i32(ip), dev_i32(ix)
    plan = g.gnn_plan_create(ip_d, ix_d)
    X = dev_feat(_feats(rng, 40, 4, "f32"), "f32")
    _, arg = g.gnn_reduce_fwd(plan, ip_d, ix_d, X)
    with pytest.raises(g.GnnError):
        g.gnn_reduce_bwd(plan, ip_d, ix_d, X, arg)


def test_rows_sorted_flag_and_unsorted_rows(g):
    """A plan records whether rows are sorted; rows in any order give the same
    exact result (the smallest winning source), through the general path."""
    rng = np.random.default_rng(21)
    n, F = 900, 32
    ip, ix = _graph(rng, n, 12, hub_deg=2000)
    X = _feats(rng, n, F, "f32")
    ixs = ix.copy()
    for i in range(n):                       # shuffle every row
        seg = ixs[ip[i]:ip[i + 1]]
        rng.shuffle(seg)
    assert not np.array_equal(ixs, ix)
    sorted_plan = g.gnn_plan_create(dev_i32(ip), dev_i32(ix))
    assert g.gnn_plan_export(sorted_plan)["rows_sorted"] == 1
    ip_d, ixs_d = dev_i32(ip), dev_i32(ixs)
    for plan in (None, g.gnn_plan_create(ip_d, ixs_d, light_threshold=16, chunk=8, waves_per_group=4)):
        if plan is not None:
            assert g.gnn_plan_export(plan)["rows_sorted"] == 0
        for op in ("max", "min"):
            for msg in ("src", "diff"):
                out, arg = g.gnn_reduce_fwd(plan, ip_d, ixs_d, dev_feat(X, "f32"), op, msg)
                ro, ra = _ref(ip, ixs, X, op, msg, "f32")
                assert np.array_equal(arg.cpu().numpy(), ra), (op, msg)
                assert np.array_equal(_bits(out.cpu().numpy()), _bits(ro)), (op, msg)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_reduce_infinities(g, dtype):
    """Rows whose messages are all -inf (max) or all +inf (min) still pick the
    smallest source; mixed rows pick the finite extreme."""
    rng = np.random.default_rng(22)
    n, F = 800, 16
    ip, ix = _graph(rng, n, 6, hub_deg=1200)
    levels = np.array([-np.inf, -1.0, 0.0, 2.0, np.inf], np.float32)
    X = rng.choice(levels, (n, F), p=[0.4, 0.1, 0.05, 0.05, 0.4])
    ip_d, ix_d = dev_i32(ip), dev_i32(ix)
    for plan in (None, g.gnn_plan_create(ip_d, ix_d, light_threshold=4, chunk=3, waves_per_group=2),
                 g.gnn_plan_create(ip_d, ix_d)):
        for op in ("max", "min"):
            out, arg = g.gnn_reduce_fwd(plan, ip_d, ix_d, dev_feat(X, dtype), op, "src")
            ro, ra = _ref(ip, ix, X, op, "src", dtype)
            assert np.array_equal(arg.cpu().numpy(), ra), op
            assert np.array_equal(_bits(_gpu_out_f32(out)), _bits(ro)), op
