"""GPU parity on feature tables of more than 2^31 elements.

Rows are 2048 elements wide (attention: H = 16 heads of D = 128; reduction
and SpMM: F = 2048), and the graph has N = 2^20 + 2^14 + 5 nodes, so every
row from 2^20 on starts past element 2^31 of its table: reading, gathering
or writing those rows needs 64-bit offsets everywhere. Each row i hears from
N-1-i (the first 2^14 + 5 rows gather rows past 2^31, the last ones are
written past it), from one pseudo-random source, and from itself; 32 aligned
16-node blocks past row 2^20 are complete (dense 16x16 tiles for the MFMA
path); node N-1 hears from 3,000 sources and node 2^20 + 1 sends to 3,000
destinations (heavy chunk groups on both sides of the backward).

Inputs are drawn on the device from a seeded torch generator. The oracle
cannot hold the whole tables (a 2.2G-element fp64 table is 17 GB), so each
check runs it on the subgraph that determines the sampled outputs: the
sampled rows and sources, every destination of a sampled source, and all
entries of those rows, with the node ids relabelled in increasing order (so
in-row order is kept). A sampled source's destinations then have their full
rows, which is all its gradient depends on."""
import numpy as np
import pytest

import oracle
from _gpu import check, say
from _helpers import dependency_subgraph

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

ROW = 2048                     # elements per node row
HI = (1 << 31) // ROW          # first node whose row starts past element 2^31
N = HI + (1 << 14) + 5
DENSE_BLOCKS = np.arange(HI // 16 + 8, HI // 16 + 40)      # complete 16-node blocks
HUB_IN, HUB_OUT, HUB_DEG = N - 1, HI + 1, 3000


@pytest.fixture(scope="module")
def g():
    import io_aware_sparse_amd as g
    g.lib()
    return g


@pytest.fixture(scope="module")
def graph(g):
    """The edge list, its CSR built on the device and checked bit for bit
    against the oracle's, and the oracle's transposed adjacency."""
    import torch
    i = np.arange(N, dtype=np.int64)
    rng = np.random.default_rng(2024)
    blk = (DENSE_BLOCKS[:, None] * 16 + np.arange(16)[None, :]).ravel()
    bi, bj = np.meshgrid(np.arange(16), np.arange(16), indexing="ij")
    dense_dst = (DENSE_BLOCKS[:, None, None] * 16 + bi[None]).ravel()
    dense_src = (DENSE_BLOCKS[:, None, None] * 16 + bj[None]).ravel()
    src = np.concatenate([N - 1 - i, (i * 7919 + 13) % N, dense_src,
                          rng.choice(N, HUB_DEG, replace=False), np.full(HUB_DEG, HUB_OUT)])
    dst = np.concatenate([i, i, dense_dst, np.full(HUB_DEG, HUB_IN), rng.choice(N, HUB_DEG, replace=False)])
    src, dst = src.astype(np.int32), dst.astype(np.int32)
    rp, rx = oracle.csr_build(src, dst, N)
    ip, ix = g.gnn_csr_build(torch.from_numpy(src).cuda(), torch.from_numpy(dst).cuda(), N)
    assert np.array_equal(ip.cpu().numpy(), rp) and np.array_equal(ix.cpu().numpy(), rx)
    cip, cix = oracle.csc(rp, rx, N)
    assert int(np.diff(rp)[HUB_IN]) > 512 and int(np.diff(cip)[HUB_OUT]) > 512
    # sampled rows and sources: the first rows (they gather rows past 2^31), the
    # rows past 2^31, two dense blocks, the hubs and a seeded spread
    pick = np.random.default_rng(7)
    lo = pick.choice(N - HI, 48, replace=False)
    hi = HI + pick.choice(N - HI, 48, replace=False)
    spread = pick.choice(N, 48, replace=False)
    rows = np.unique(np.concatenate([lo, hi, spread, blk[:32], [0, HI - 1, HI, N - 1, HUB_IN, HUB_OUT]]))
    srcs = np.unique(np.concatenate([hi, lo, spread[:24], blk[16:48], [HUB_OUT, N - 1, HI]]))
    say(f"N={N} E={rx.size}: rows past element 2^31 from {HI}; {rows.size} rows, {srcs.size} sources sampled")
    return dict(ip=ip, ix=ix, rp=rp, rx=rx, cip=cip, cix=cix, rows=rows, srcs=srcs)


def _subgraph(G):
    return dependency_subgraph(*(G[k] for k in ("rp", "rx", "cip", "cix", "rows", "srcs")))


def _take(x, U):
    """Rows U of a device table, widened to fp32 on the host."""
    import torch
    return x.index_select(0, torch.from_numpy(U).cuda()).float().cpu().numpy()


def _host(x, ids):
    return _take(x, ids).astype(np.float64)


def _randn(gen, shape, dtype):
    import torch
    return torch.randn(shape, generator=gen, device="cuda", dtype=dtype)


@pytest.mark.parametrize("tau", [0.0, 0.75])
def test_gt_beyond_int32_offsets(g, graph, tau):
    """GT forward and backward in bf16 (H = 16, D = 128), default plan and
    tiled plan (tau = 0.75: the complete blocks become tiles)."""
    import torch
    H, D = 16, 128
    say(f"GT bf16 16x128 on {N} nodes (tables of {N * ROW / 2 ** 31:.3f} x 2^31 elements), tile density {tau}")
    gen = torch.Generator(device="cuda").manual_seed(11)
    q, k, v, go = (_randn(gen, (N, H, D), torch.bfloat16) for _ in range(4))
    plan = g.gnn_plan_create(graph["ip"], graph["ix"], want_csc=True, tile_density=tau)
    if tau > 0:
        info = g.gnn_plan_export(plan)
        say(f"  tiles {info['n_tiles']}, tiled row blocks {info['n_trb']}, column blocks {info['n_tcb']}")
        assert info["n_tiles"] >= DENSE_BLOCKS.size and info["n_trb"] >= DENSE_BLOCKS.size
    O, L = g.gnn_attn_fwd(plan, graph["ip"], graph["ix"], q, k, v)
    dq, dk, dv = g.gnn_attn_bwd(plan, graph["ip"], graph["ix"], q, k, v, O, go, L)
    torch.cuda.synchronize()
    s = _subgraph(graph)
    U = s["U"]
    Q, K, V, dO = (_take(x, U).reshape(U.size, H, D) for x in (q, k, v, go))
    rows, srcs = graph["rows"], graph["srcs"]
    ref = oracle.gt_fwd(s["sp"], s["sx"], Q, K, V, rows=s["rows"])
    check("O", _host(O, rows).reshape(-1, H, D), ref["O"], ref["SO"], "bf16")
    check("LSE", L.index_select(0, torch.from_numpy(rows).cuda()).cpu().numpy(), ref["LSE"], ref["SL"], "f32")
    rb = oracle.gt_bwd(s["sp"], s["sx"], Q, K, V, dO, rows=s["rows"], srcs=s["srcs"])
    check("dQ", _host(dq, rows).reshape(-1, H, D), rb["dQ"], rb["SdQ"], "bf16")
    check("dK", _host(dk, srcs).reshape(-1, H, D), rb["dK"], rb["SdK"], "bf16")
    check("dV", _host(dv, srcs).reshape(-1, H, D), rb["dV"], rb["SdV"], "bf16")
    del q, k, v, go, O, L, dq, dk, dv
    torch.cuda.empty_cache()


def test_gatv2_beyond_int32_offsets(g, graph):
    """GATv2 forward and backward in fp32 (H = 16, D = 128)."""
    import torch
    H, D = 16, 128
    say(f"GATv2 fp32 16x128 on {N} nodes")
    gen = torch.Generator(device="cuda").manual_seed(12)
    xd, xs, go = (_randn(gen, (N, H, D), torch.float32) for _ in range(3))
    at = _randn(gen, (H, D), torch.float32) / np.sqrt(D)
    plan = g.gnn_plan_create(graph["ip"], graph["ix"], want_csc=True)
    O, L = g.gatv2_attn_fwd(plan, graph["ip"], graph["ix"], xd, xs, at, negative_slope=0.2)
    gxd, gxs, _, gda = g.gatv2_attn_bwd(plan, graph["ip"], graph["ix"], xd, xs, at, go, L)
    torch.cuda.synchronize()
    s = _subgraph(graph)
    U = s["U"]
    XD, XS, dO = (_take(x, U).reshape(U.size, H, D) for x in (xd, xs, go))
    att = at.cpu().numpy()
    rows, srcs = graph["rows"], graph["srcs"]
    ref = oracle.gatv2_fwd(s["sp"], s["sx"], XD, XS, att, slope=0.2, rows=s["rows"])
    check("O", _host(O, rows).reshape(-1, H, D), ref["O"], ref["SO"], "f32")
    rb = oracle.gatv2_bwd(s["sp"], s["sx"], XD, XS, att, dO, slope=0.2, rows=s["rows"], srcs=s["srcs"],
                          want_da=False)
    check("dXD", _host(gxd, rows).reshape(-1, H, D), rb["dXD"], rb["SdXD"], "f32")
    check("dXS", _host(gxs, srcs).reshape(-1, H, D), rb["dXS"], rb["SdXS"], "f32")
    assert torch.isfinite(gda).all()
    del xd, xs, go, O, L, gxd, gxs, gda
    torch.cuda.empty_cache()


def test_reduce_beyond_int32_offsets(g, graph):
    """Max of sources and min of differences in bf16 (F = 2048): values and
    winners bit for bit on the sampled rows, the gradient on the sampled
    sources."""
    import torch
    say(f"max / min reduction bf16 F={ROW} on {N} nodes")
    gen = torch.Generator(device="cuda").manual_seed(13)
    xd, god = (_randn(gen, (N, ROW), torch.bfloat16) for _ in range(2))
    plan = g.gnn_plan_create(graph["ip"], graph["ix"], want_csc=True)
    s = _subgraph(graph)
    U = s["U"]
    X, dOut = _take(xd, U), _take(god, U)
    rows, srcs = graph["rows"], graph["srcs"]
    for op, msg in (("max", "src"), ("min", "diff")):
        out, arg = g.gnn_reduce_fwd(plan, graph["ip"], graph["ix"], xd, op, msg)
        dX = g.gnn_reduce_bwd(plan, graph["ip"], graph["ix"], god, arg, msg)
        torch.cuda.synchronize()
        ref = oracle.segment_reduce(s["sp"], s["sx"], X, op, msg, rows=s["need"])
        at = {int(li): r for r, li in enumerate(s["need"])}
        ri = np.array([at[int(li)] for li in s["rows"]])
        want_arg = np.where(ref["arg"][ri] >= 0, U[np.maximum(ref["arg"][ri], 0)], -1)
        want_out = oracle.round_bf16(ref["out"][ri]) if msg == "diff" else ref["out"][ri]
        got_arg = arg.index_select(0, torch.from_numpy(rows).cuda()).cpu().numpy()
        got_out = _take(out, rows)
        ok_arg = np.array_equal(got_arg, want_arg)
        ok_out = np.array_equal(got_out.view(np.uint32), np.ascontiguousarray(want_out, np.float32).view(np.uint32))
        say(f"  {op} {msg}: {rows.size} rows, winners equal {ok_arg}, values equal {ok_out}")
        assert ok_arg and ok_out, (op, msg)
        rdX, S = oracle.segment_reduce_bwd(s["sp"], s["sx"], dOut[s["need"]], ref["arg"], msg,
                                           n_nodes=U.size, want_scale=True, rows=s["need"])
        check(f"dX {op} {msg}", _host(dX, srcs), rdX[s["srcs"]], S[s["srcs"]], "bf16")
        del out, arg, dX
    del xd, god
    torch.cuda.empty_cache()


def test_spmm_beyond_int32_offsets(g, graph):
    """Mean-normalised SpMM and its transpose in bf16 (F = 2048): sampled rows
    and sources."""
    import torch
    say(f"SpMM (mean) bf16 F={ROW} on {N} nodes")
    gen = torch.Generator(device="cuda").manual_seed(14)
    xd, god = (_randn(gen, (N, ROW), torch.bfloat16) for _ in range(2))
    plan = g.gnn_plan_create(graph["ip"], graph["ix"], want_csc=True)
    g.gnn_spmm_prepare(plan, "mean")
    Y = g.gnn_spmm(plan, graph["ip"], graph["ix"], xd)
    dX = g.gnn_spmm(plan, graph["ip"], graph["ix"], god, transpose=True)
    torch.cuda.synchronize()
    s = _subgraph(graph)
    U = s["U"]
    ref = oracle.spmm(s["sp"], s["sx"], _take(xd, U), "mean", rows=s["rows"])
    check("Y", _host(Y, graph["rows"]), ref["Y"], ref["S"], "bf16")
    ref = oracle.spmm(s["sp"], s["sx"], _take(god, U), "mean", transpose=True, rows=s["srcs"])
    check("dX", _host(dX, graph["srcs"]), ref["Y"], ref["S"], "bf16")
    del xd, god, Y, dX
    torch.cuda.empty_cache()
