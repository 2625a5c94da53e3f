"""Degenerate inputs through every entry point on the GPU.

The empty graph (N = 0, E = 0), with and without a plan: every call returns
GNN_OK and writes nothing. A graph whose rows are all empty (N = 37, E = 0,
no self-loops), with no plan, a plan and a tiled plan: attention O = 0 and
LSE = -inf with zero gradients (the softmax over an empty neighbourhood is
taken as empty), GATv2 likewise and d_att = 0, the max / min reduction 0
with no winner (-1) and a zero gradient, the SpMM and its transpose 0, and
the reorderings valid permutations of the nodes."""
import numpy as np
import pytest

import oracle
from _gpu import dev_i32, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def g():
    import io_aware_sparse_amd as g
    g.lib()
    return g


def _all_calls(g, plan, ip, ix, n, dtype):
    """Run every compute entry point; returns their outputs (torch tensors).
    Every output buffer starts filled with NaN (indices with a sentinel), so
    an element a call leaves unwritten cannot pass for a zero."""
    import torch
    H, D = 2, 32
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    gen = torch.Generator(device="cuda").manual_seed(3)
    q, k, v, go = (torch.randn((n, H, D), generator=gen, device="cuda", dtype=tdt) for _ in range(4))
    att = torch.randn((H, D), generator=gen, device="cuda")
    nan = lambda shape, dt=tdt: torch.full(shape, float("nan"), dtype=dt, device="cuda")   # noqa: E731
    feat, stat, rows = (n, H, D), (n, H), (n, H * D)
    out = {}
    out["O"], out["L"] = g.gnn_attn_fwd(plan, ip, ix, q, k, v, O=nan(feat), LSE=nan(stat, torch.float32))
    if plan is not None:
        out["dQ"], out["dK"], out["dV"] = g.gnn_attn_bwd(plan, ip, ix, q, k, v, out["O"], go, out["L"],
                                                         dQ=nan(feat), dK=nan(feat), dV=nan(feat))
        O2, L2 = nan(feat), nan(stat, torch.float32)
        g.gnn_attn_fwd_noalloc(plan, ip, ix, q, k, v, O2, L2)
        out["O_noalloc"], out["L_noalloc"] = O2, L2
    out["GO"], out["GL"] = g.gatv2_attn_fwd(plan, ip, ix, q, k, att, O=nan(feat), LSE=nan(stat, torch.float32))
    if plan is not None:
        out["dXD"], out["dXS"], _, out["d_att"] = g.gatv2_attn_bwd(
            plan, ip, ix, q, k, att, go, out["GL"], dXD=nan(feat), dXS=nan(feat), d_att=nan((H, D), torch.float32))
    X = q.reshape(rows)
    out["X"] = X
    for op, msg in (("max", "src"), ("min", "diff")):
        r, a = g.gnn_reduce_fwd(plan, ip, ix, X, op, msg, out=nan(rows),
                                arg=torch.full(rows, 12345, dtype=torch.int32, device="cuda"))
        out[f"red_{op}"], out[f"arg_{op}"] = r, a
        if plan is not None:
            out[f"dX_{op}"] = g.gnn_reduce_bwd(plan, ip, ix, go.reshape(rows), a, msg, dX=nan(rows))
    if plan is not None:
        g.gnn_spmm_prepare(plan, "gcn")
        out["Y"] = g.gnn_spmm(plan, ip, ix, X, Y=nan(rows))
        out["YT"] = g.gnn_spmm(plan, ip, ix, X, transpose=True, Y=nan(rows))
    for method in ("degree", "rcm"):
        perm = g.gnn_reorder(ip, ix, method)
        out[f"perm_{method}"] = perm
        pip, pix = g.gnn_permute_graph(ip, ix, perm)
        out[f"pip_{method}"] = pip
        out[f"rows_{method}"] = g.gnn_permute_rows(X, perm, dst=nan(rows))
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_empty_graph(g, dtype):
    import torch
    say("empty graph (N = 0)", dtype)
    none = np.zeros(0, np.int32)
    ip, ix = g.gnn_csr_build(dev_i32(none), dev_i32(none), 0)
    assert ip.cpu().numpy().tolist() == [0] and ix.numel() == 0
    for plan in (None, g.gnn_plan_create(ip, ix, want_csc=True)):
        out = _all_calls(g, plan, ip, ix, 0, dtype)
        for name, x in out.items():
            if name.startswith("pip_"):
                assert x.cpu().numpy().tolist() == [0], name
            elif name == "d_att":
                assert torch.all(x == 0).item(), name
            else:
                assert x.shape[0] == 0, (name, tuple(x.shape))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("plan_kind", ["none", "plan", "tiles"])
def test_all_rows_empty(g, dtype, plan_kind):
    import torch
    n = 37
    say("all rows empty", dtype, plan_kind)
    none = np.zeros(0, np.int32)
    ip, ix = g.gnn_csr_build(dev_i32(none), dev_i32(none), n, add_self_loops=False)
    assert np.array_equal(ip.cpu().numpy(), np.zeros(n + 1, np.int32)) and ix.numel() == 0
    plan = None if plan_kind == "none" else \
        g.gnn_plan_create(ip, ix, want_csc=True, tile_density=0.75 if plan_kind == "tiles" else 0.0)
    out = _all_calls(g, plan, ip, ix, n, dtype)
    for name in ("O", "GO", "dQ", "dK", "dV", "dXD", "dXS", "d_att", "dX_max", "dX_min", "Y", "YT", "O_noalloc",
                 "red_max", "red_min"):
        if name in out:
            assert torch.all(out[name].float() == 0).item(), name
    for name in ("L", "GL", "L_noalloc"):
        if name in out:
            assert torch.all(torch.isneginf(out[name])).item(), name
    for name in ("arg_max", "arg_min"):
        assert torch.all(out[name] == -1).item(), name
    ref = oracle.gt_fwd(np.zeros(n + 1, np.int64), none, np.ones((n, 2, 32)), np.ones((n, 2, 32)),
                        np.ones((n, 2, 32)))
    assert np.all(ref["O"] == 0) and np.all(np.isneginf(ref["LSE"]))          # the oracle's reading agrees
    for method in ("degree", "rcm"):
        perm = out[f"perm_{method}"].cpu().numpy()
        assert np.array_equal(np.sort(perm), np.arange(n)), method
        assert np.array_equal(out[f"pip_{method}"].cpu().numpy(), np.zeros(n + 1, np.int32)), method
        want = out["X"].index_select(0, out[f"perm_{method}"].long())
        assert torch.equal(out[f"rows_{method}"], want), method
