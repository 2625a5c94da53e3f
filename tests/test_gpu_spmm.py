"""GPU parity of the cached SpMM aggregation (gnn_spmm_prepare / gnn_spmm)
against the oracle: cached weights, Y = A_w X and A_w^T X for sum, mean and
GCN weights, fp32 and bf16, rows from one 16-byte slice to several waves,
plans whose tiny threshold sends most rows through the chunked heavy path,
repeated entries and empty rows; reproducibility and the error paths."""
import numpy as np
import pytest

import oracle
from _gpu import TOL, check, dev_feat, dev_i32, host, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def g():
    import io_aware_sparse_amd as g
    g.lib()
    return g


def _graph(rng, n, mean_deg, hub_deg=0, empty=0.03):
    deg = rng.poisson(mean_deg, n)
    if hub_deg:
        deg[rng.choice(n, 3, replace=False)] = hub_deg
    deg[rng.random(n) < empty] = 0
    rows = [np.sort(np.concatenate([rng.integers(0, n, d), rng.integers(0, n, int(d > 4))])) for d in deg]
    ip = np.concatenate([[0], np.cumsum([r.size for r in rows])]).astype(np.int32)
    ix = np.concatenate(rows).astype(np.int32)
    return ip, ix


def _feats(rng, n, F, dtype):
    x = rng.standard_normal((n, F)).astype(np.float32)
    return oracle.round_bf16(x) if dtype == "bf16" else x


def _plan(g, ip_d, ix_d, kind):
    if kind == "tiny":
        return g.gnn_plan_create(ip_d, ix_d, light_threshold=3, chunk=2, waves_per_group=2, want_csc=True)
    return g.gnn_plan_create(ip_d, ix_d, want_csc=True)


@pytest.mark.parametrize("norm", ["sum", "mean", "gcn"])
def test_cached_weights(g, norm):
    rng = np.random.default_rng(1)
    n = 400
    ip, ix = _graph(rng, n, 6, hub_deg=700)
    plan = g.gnn_plan_create(dev_i32(ip), dev_i32(ix), want_csc=True)
    g.gnn_spmm_prepare(plan, norm)
    d = g.gnn_plan_export(plan, arrays=True)
    assert d["spmm_norm"] == g.NORMS[norm]
    w = oracle.spmm_weights(ip, ix, norm)
    assert np.all((d["spmm_w"] == 0) == (w == 0))
    nz = w > 0
    assert np.max(np.abs(d["spmm_w"][nz] - w[nz]) / w[nz]) < 1e-6
    rows = np.repeat(np.arange(n), np.diff(ip))
    o = np.lexsort((rows, ix))                       # CSR entries in transposed order (source, then row)
    wo = w[o]
    assert np.all((d["spmm_cw"] == 0) == (wo == 0))
    assert np.max(np.abs(d["spmm_cw"][wo > 0] - wo[wo > 0]) / wo[wo > 0]) < 1e-6
    if norm == "gcn":
        assert (w == 0).any()                        # the graph has sources without entries


CASES = [("f32", 4), ("f32", 96), ("f32", 128), ("f32", 320), ("bf16", 8), ("bf16", 128), ("bf16", 200), ("bf16", 1032)]


@pytest.mark.parametrize("dtype,F", CASES)
@pytest.mark.parametrize("plan_kind", ["tiny", "default"])
def test_spmm_parity(g, dtype, F, plan_kind):
    rng = np.random.default_rng(F + len(plan_kind))
    n = 600
    ip, ix = _graph(rng, n, 9, hub_deg=1500)
    X = _feats(rng, n, F, dtype)
    ip_d, ix_d = dev_i32(ip), dev_i32(ix)
    plan = _plan(g, ip_d, ix_d, plan_kind)
    Xd = dev_feat(X, dtype)
    for norm in ("sum", "mean", "gcn"):
        g.gnn_spmm_prepare(plan, norm)
        for tr in (False, True):
            Y = g.gnn_spmm(plan, ip_d, ix_d, Xd, transpose=tr)
            ref = oracle.spmm(ip, ix, X, norm, transpose=tr)
            check(f"spmm {dtype} F={F} {plan_kind} {norm} transpose={tr}", host(Y), ref["Y"], ref["S"], dtype)
            Y2 = g.gnn_spmm(plan, ip_d, ix_d, Xd, transpose=tr)
            assert np.array_equal(host(Y2), host(Y)), "not reproducible"


@pytest.mark.parametrize("dtype,F", [("f32", 128), ("f32", 64), ("bf16", 128), ("bf16", 256)])
@pytest.mark.parametrize("threshold", [512, 200])
def test_spmm_long_light_rows(g, dtype, F, threshold):
    """Light rows of more than 128 entries head the packed order and get a wave
    each (2 or 4 rows per wave for the rest): rows of 100-700 entries and 150
    popular sources put such rows on both sides of 128 and of the light
    threshold, in the product and in the transposed product."""
    rng = np.random.default_rng(F + threshold)
    n = 3000
    deg = rng.poisson(6, n)
    deg[rng.choice(n, 200, replace=False)] = rng.integers(100, 700, 200)
    popular = rng.choice(n, 150, replace=False)
    rows = []
    for d in deg:
        src = rng.integers(0, n, d)
        pick = rng.random(d) < 0.3
        src[pick] = popular[rng.integers(0, popular.size, int(pick.sum()))]
        rows.append(np.sort(src))
    ip = np.concatenate([[0], np.cumsum(deg)]).astype(np.int32)
    ix = np.concatenate(rows).astype(np.int32)
    indeg, outdeg = np.diff(ip), np.bincount(ix, minlength=n)
    X = _feats(rng, n, F, dtype)
    ip_d, ix_d = dev_i32(ip), dev_i32(ix)
    plan = g.gnn_plan_create(ip_d, ix_d, light_threshold=threshold, want_csc=True)
    d = g.gnn_plan_export(plan, arrays=True)
    n_long = int(((indeg > 128) & (indeg <= threshold)).sum())
    c_n_long = int(((outdeg > 128) & (outdeg <= threshold)).sum())
    say(f"n={n} E={ip[-1]} threshold={threshold}: {n_long} long light rows, {c_n_long} long light sources")
    assert n_long > 0 and c_n_long > 0
    assert d["n_long_light"] == n_long and d["c_n_long_light"] == c_n_long
    assert np.all(indeg[d["light_by_degree"][:n_long]] > 128)          # the head of the packed order
    assert np.all(indeg[d["light_by_degree"][n_long:]] <= 128)
    assert np.all(outdeg[d["c_light_by_degree"][:c_n_long]] > 128)
    Xd = dev_feat(X, dtype)
    for norm in ("gcn", "sum"):
        g.gnn_spmm_prepare(plan, norm)
        for tr in (False, True):
            Y = g.gnn_spmm(plan, ip_d, ix_d, Xd, transpose=tr)
            ref = oracle.spmm(ip, ix, X, norm, transpose=tr)
            check(f"spmm long rows {dtype} F={F} T={threshold} {norm} transpose={tr}", host(Y), ref["Y"],
                  ref["S"], dtype)
            Y2 = g.gnn_spmm(plan, ip_d, ix_d, Xd, transpose=tr)
            assert np.array_equal(host(Y2), host(Y)), "not reproducible"


def _tile_graph(kind):
    """CSR arrays (rows sorted, repeated entries kept) for the tiled-plan tests."""
    if kind == "blocks":
        rng = np.random.default_rng(401)
        n = 1000                                     # a ragged last block of 8 rows
        a = rng.random((n, n)) < 0.01
        for b0 in range(0, n - 15, 16):
            if rng.random() < 0.6:
                a[b0:b0 + 16, b0:b0 + 16] |= rng.random((16, 16)) < rng.uniform(0.6, 1.0)
            if rng.random() < 0.3:                   # dense off-diagonal blocks: several tiles per row
                c0 = 16 * int(rng.integers(1, n // 16))          # and per column block
                a[b0:b0 + 16, c0:c0 + 16] |= rng.random((16, 16)) < rng.uniform(0.6, 1.0)
        a[:, 7] = True                               # a heavy source: its column block is never tiled
        a[333, :] = True                             # a heavy row: its row block is never tiled
        a[900:916, :] = False                        # empty rows inside a block
        dst, src = np.nonzero(a)
        dup = rng.choice(src.size, src.size // 20, replace=False)   # repeated entries, tiled and not
        dst, src = np.concatenate([dst, dst[dup]]), np.concatenate([src, src[dup]])
    else:
        import workloads
        wl = workloads.make(kind, 2048, features=False)
        n, dst, src = wl.n_nodes, wl.dst.astype(np.int64), wl.src.astype(np.int64)
    order = np.lexsort((src, dst))
    dst, src = dst[order], src[order]
    ip = np.concatenate([[0], np.cumsum(np.bincount(dst, minlength=n))]).astype(np.int32)
    return ip, src.astype(np.int32), n


@pytest.mark.parametrize("dtype,F", [("f32", 16), ("f32", 32), ("f32", 64), ("bf16", 16), ("bf16", 48), ("bf16", 128),
                                     ("bf16", 256)])
@pytest.mark.parametrize("kind,tau,T", [("spmm_comm16_n1m_deg27", 0.75, 512), ("blocks", 0.5, 60)])
def test_spmm_tiled_plan(g, dtype, F, kind, tau, T):
    """Plans with a tile census: tiled blocks run on the 16x16 block kernel
    (MFMA tile products plus the blocks' residual entries), the other light
    rows and the heavy rows on the CSR kernel; rows of more than 256 bytes
    (bf16, F = 256) stay on the CSR kernel. Both products, three norms."""
    rng = np.random.default_rng(F + int(100 * tau))
    ip, ix, n = _tile_graph(kind)
    ip_d, ix_d = dev_i32(ip), dev_i32(ix)
    plan = g.gnn_plan_create(ip_d, ix_d, light_threshold=T, chunk=32, tile_density=tau, want_csc=True)
    info = g.gnn_plan_export(plan)
    say(f"{kind}: n={n} E={ip[-1]} tiles={info['n_tiles']} tiled row blocks={info['n_trb']} "
        f"tiled column blocks={info['n_tcb']} residual={info['n_residual']}")
    assert info["n_tiles"] > 0 and info["n_trb"] > 0 and info["n_tcb"] > 0
    if kind == "blocks":                              # blocks with several tiles, both ways
        d = g.gnn_plan_export(plan, arrays=True)
        assert np.diff(d["tile_ptr"]).max() >= 2 and np.diff(d["ctile_ptr"]).max() >= 2
    block_path = F * (2 if dtype == "bf16" else 4) <= 256
    X = _feats(rng, n, F, dtype)
    Xd = dev_feat(X, dtype)
    for norm in ("gcn", "mean", "sum"):
        g.gnn_spmm_prepare(plan, norm)
        for tr in (False, True):
            g.gnn_plan_set_timing(plan, True)
            Y = g.gnn_spmm(plan, ip_d, ix_d, Xd, transpose=tr)
            ran = g.gnn_plan_timing_read(plan)
            g.gnn_plan_set_timing(plan, False)
            assert (("spmm_t_wsb" if tr else "spmm_wsb") in ran) == block_path, ran
            ref = oracle.spmm(ip, ix, X, norm, transpose=tr)
            check(f"tiled spmm {kind} {dtype} F={F} {norm} transpose={tr}", host(Y), ref["Y"], ref["S"], dtype)
            Y2 = g.gnn_spmm(plan, ip_d, ix_d, Xd, transpose=tr)
            assert np.array_equal(host(Y2), host(Y)), "not reproducible"


def test_spmm_errors_and_empty(g):
    import torch
    rng = np.random.default_rng(3)
    n = 50
    ip, ix = _graph(rng, n, 3)
    ip_d, ix_d = dev_i32(ip), dev_i32(ix)
    X = dev_feat(_feats(rng, n, 4, "f32"), "f32")
    plan = g.gnn_plan_create(ip_d, ix_d)
    with pytest.raises(g.GnnError):                  # not prepared
        g.gnn_spmm(plan, ip_d, ix_d, X)
    g.gnn_spmm_prepare(plan, "gcn")
    with pytest.raises(g.GnnError):                  # no transposed adjacency in this plan
        g.gnn_spmm(plan, ip_d, ix_d, X, transpose=True)
    Y = g.gnn_spmm(plan, ip_d, ix_d, X)
    empty = np.diff(ip) == 0
    assert empty.any() and torch.all(Y[torch.from_numpy(empty).cuda()] == 0).item()
