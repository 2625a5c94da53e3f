"""GPU parity at the largest accepted edge count.

The library accepts E <= 2^31 - 2^21 entries (int32 positions with headroom
for a step of edges past the end). The graph has N = 2^20 nodes and exactly
that many entries: row i lists the sources (i + 513 k) mod N for
k = 0 .. 2045 (k = 0 is the self-loop the CSR build adds; 513 is odd, so the
sources of a row are distinct), 2,046 entries per row, so entry positions run
up to 2^31 - 2^21 and every row is heavy at the default threshold. The input
list (k = 1 .. 2045, destination-major) is built on the device.

The structure is known in closed form: indptr is checked in full, the rows
of the sampled nodes entry by entry, and every row for strictly increasing
sources. Outputs are compared with the oracle on the sampled rows and
sources, run on the subgraph of the rows they depend on (sampled rows and
sources and every destination of a sampled source, with their full rows);
features are small (H = 1, D = 16, fp32: 64 MB tables), so every kernel
family runs on the full graph: GT forward and backward on the default plan
(all rows heavy) and on a plan whose threshold makes them light, the GATv2
forward, the max reduction and the SpMM with its transpose."""
import numpy as np
import pytest

import oracle
from _gpu import check, say
from _helpers import stride_dests, stride_rows

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

N = 1 << 20
STEP = 513
DEG = 2046
E = N * DEG
assert E == (1 << 31) - (1 << 21)


def _rows_of(ids):
    return stride_rows(ids, N, STEP, DEG)


def _dests_of(j):
    return stride_dests(j, N, STEP, DEG)


@pytest.fixture(scope="module")
def g():
    import io_aware_sparse_amd as g
    g.lib()
    return g


@pytest.fixture(scope="module")
def graph(g):
    import torch
    say(f"edge-limit graph: N={N}, E={E} (2^31 - 2^21), {DEG} entries per row")
    i = torch.arange(N, dtype=torch.int32, device="cuda")
    k = torch.arange(1, DEG, dtype=torch.int32, device="cuda")
    dst = i[:, None].expand(N, DEG - 1).reshape(-1)
    src = ((i[:, None] + STEP * k[None, :]) % N).reshape(-1)
    ip, ix = g.gnn_csr_build(src, dst, N)
    del src, dst, i, k
    torch.cuda.synchronize()
    assert ix.numel() == E
    want_ip = (np.arange(N + 1, dtype=np.int64) * DEG).astype(np.int32)
    assert np.array_equal(ip.cpu().numpy(), want_ip)
    mono = bool((ix.view(N, DEG).diff(dim=1) > 0).all().item())
    assert mono, "rows not strictly increasing"
    pick = np.random.default_rng(3)
    rows = np.unique(np.concatenate([pick.choice(N, 40, replace=False), [0, 1, N - 2, N - 1]]))
    srcs = np.unique(np.concatenate([pick.choice(N, 4, replace=False), [0, N - 1]]))
    got = ix.view(N, DEG).index_select(0, torch.from_numpy(rows).cuda()).cpu().numpy()
    assert np.array_equal(got, _rows_of(rows))
    # subgraph over the global ids: full rows for the rows the samples depend on
    need = np.unique(np.concatenate([rows, srcs] + [_dests_of(j) for j in srcs]))
    deg = np.zeros(N, np.int64)
    deg[need] = DEG
    sp = np.concatenate([[0], np.cumsum(deg)])
    sx = _rows_of(need).ravel()
    say(f"  CSR checked (indptr in full, {rows.size} rows entry by entry, all rows increasing); "
        f"oracle subgraph of {need.size} rows, {sx.size} entries")
    return dict(ip=ip, ix=ix, rows=rows, srcs=srcs, sp=sp, sx=sx, need=need)


def _host(x, ids):
    import torch
    return x.index_select(0, torch.from_numpy(np.asarray(ids, np.int64)).cuda()).double().cpu().numpy()


@pytest.mark.parametrize("threshold", [512, 4096])
def test_gt_at_edge_limit(g, graph, threshold):
    """GT forward and backward, every row heavy (threshold 512: four chunks of
    512 entries, one group) or light (threshold 4096)."""
    import torch
    H, D = 1, 16
    rng = np.random.default_rng(31)
    Q, K, V, dO = (rng.standard_normal((N, H, D)).astype(np.float32) for _ in range(4))
    q, k, v, go = (torch.from_numpy(x).cuda() for x in (Q, K, V, dO))
    plan = g.gnn_plan_create(graph["ip"], graph["ix"], light_threshold=threshold, want_csc=True)
    info = g.gnn_plan_export(plan)
    say(f"GT at the edge limit, threshold {threshold}: heavy {info['n_heavy']}, light {info['n_light']}, "
        f"source side heavy {info['c_n_heavy']}")
    assert (info["n_heavy"], info["c_n_heavy"]) == ((N, N) if threshold < DEG else (0, 0))
    O, L = g.gnn_attn_fwd(plan, graph["ip"], graph["ix"], q, k, v)
    dq, dk, dv = g.gnn_attn_bwd(plan, graph["ip"], graph["ix"], q, k, v, O, go, L)
    torch.cuda.synchronize()
    rows, srcs = graph["rows"], graph["srcs"]
    ref = oracle.gt_fwd(graph["sp"], graph["sx"], Q, K, V, rows=rows)
    check("O", _host(O, rows), ref["O"], ref["SO"], "f32")
    check("LSE", _host(L, rows), ref["LSE"], ref["SL"], "f32")
    rb = oracle.gt_bwd(graph["sp"], graph["sx"], Q, K, V, dO, rows=rows, srcs=srcs)
    check("dQ", _host(dq, rows), rb["dQ"], rb["SdQ"], "f32")
    check("dK", _host(dk, srcs), rb["dK"], rb["SdK"], "f32")
    check("dV", _host(dv, srcs), rb["dV"], rb["SdV"], "f32")
    del plan, O, L, dq, dk, dv
    torch.cuda.empty_cache()


def test_gatv2_reduce_spmm_at_edge_limit(g, graph):
    """GATv2 forward, max reduction (bit for bit) with its gradient, and the
    mean SpMM with its transpose, default plan."""
    import torch
    H, D = 1, 16
    rng = np.random.default_rng(32)
    XD, XS, X, dOut = (rng.standard_normal((N, H, D)).astype(np.float32) for _ in range(4))
    att = (rng.standard_normal((H, D)) / np.sqrt(D)).astype(np.float32)
    xd, xs, xx, gd = (torch.from_numpy(a).cuda() for a in (XD, XS, X, dOut))
    plan = g.gnn_plan_create(graph["ip"], graph["ix"], want_csc=True)
    rows, srcs, sp, sx, need = (graph[k] for k in ("rows", "srcs", "sp", "sx", "need"))
    say("GATv2 forward at the edge limit")
    O, _ = g.gatv2_attn_fwd(plan, graph["ip"], graph["ix"], xd, xs, torch.from_numpy(att).cuda(),
                            negative_slope=0.2)
    torch.cuda.synchronize()
    ref = oracle.gatv2_fwd(sp, sx, XD, XS, att, slope=0.2, rows=rows)
    check("O", _host(O, rows), ref["O"], ref["SO"], "f32")
    del O
    say("max reduction at the edge limit")
    out, arg = g.gnn_reduce_fwd(plan, graph["ip"], graph["ix"], xx.view(N, D), "max", "src")
    dX = g.gnn_reduce_bwd(plan, graph["ip"], graph["ix"], gd.view(N, D), arg, "src")
    torch.cuda.synchronize()
    ref = oracle.segment_reduce(sp, sx, X.reshape(N, D), "max", "src", rows=need)
    at = {int(v): r for r, v in enumerate(need)}
    ri = np.array([at[int(v)] for v in rows])
    got_arg = arg.index_select(0, torch.from_numpy(rows).cuda()).cpu().numpy()
    got_out = out.index_select(0, torch.from_numpy(rows).cuda()).cpu().numpy()
    assert np.array_equal(got_arg, ref["arg"][ri])
    assert np.array_equal(got_out.view(np.uint32), ref["out"][ri].view(np.uint32))
    rdX, S = oracle.segment_reduce_bwd(sp, sx, dOut.reshape(N, D)[need], ref["arg"], "src", n_nodes=N,
                                       want_scale=True, rows=need)
    check("dX max", _host(dX, srcs), rdX[srcs], S[srcs], "f32")
    del out, arg, dX
    say("mean SpMM at the edge limit")
    g.gnn_spmm_prepare(plan, "mean")
    Y = g.gnn_spmm(plan, graph["ip"], graph["ix"], xx.view(N, D))
    dY = g.gnn_spmm(plan, graph["ip"], graph["ix"], gd.view(N, D), transpose=True)
    torch.cuda.synchronize()
    ref = oracle.spmm(sp, sx, X.reshape(N, D), "mean", rows=rows)
    check("Y", _host(Y, rows), ref["Y"], ref["S"], "f32")
    ref = oracle.spmm(sp, sx, dOut.reshape(N, D), "mean", transpose=True, rows=srcs)
    check("dX", _host(dY, srcs), ref["Y"], ref["S"], "f32")
    del plan, Y, dY
    torch.cuda.empty_cache()
