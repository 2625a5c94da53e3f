"""Device-memory audit of the attention calls at full size.

The fused kernels never hold per-edge logits or messages: the only memory a
call may add is the plan's workspace (heavy-node partials, per-node
backward statistics, GATv2 per-node score gradients), whose size is a closed
form in the plan's counts. Checked here:

* the workspace equals that closed form after each call;
* no workspace allocation reaches E*H*2 bytes (an fp16 logit per edge and
  head would already need that much);
* the device free memory drops by no more than the workspace growth across
  a call, up to the allocator's 2 MiB pages (outputs come from torch's
  allocator and are counted separately);
* a second call with the same shapes leaves the workspace as it is and
  takes no more than one such page.
"""
import numpy as np
import pytest

import workloads
from _gpu import say

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

MIB = 1 << 20
PAGE = 2 * MIB      # granularity at which the device free memory moves


@pytest.fixture(scope="module")
def g():
    import io_aware_sparse_amd as g
    g.lib()
    _load_code_objects(g)
    return g


def _load_code_objects(g):
    """Run each attention code path once on a tiny graph. A code object is
    loaded onto the device at its first kernel launch, with its static device
    data (the allocation-free forward's 16 MiB scratch lives in the attention
    code object): a one-time cost per process, which the audits below must
    not count against the call they measure."""
    import torch
    wl = workloads.make("gt_comm16_n1m_deg27", 256, features=False)
    ip, ix = g.gnn_csr_build(torch.from_numpy(wl.src).cuda(), torch.from_numpy(wl.dst).cuda(), wl.n_nodes)
    plan = g.gnn_plan_create(ip, ix, want_csc=True, tile_density=0.75)
    assert g.gnn_plan_export(plan)["n_tiles"] > 0
    for dt, H, D in ((torch.bfloat16, 8, 64), (torch.float32, 2, 16)):
        q = torch.randn(wl.n_nodes, H, D, device="cuda").to(dt)
        O, L = g.gnn_attn_fwd(plan, ip, ix, q, q, q)
        g.gnn_attn_bwd(plan, ip, ix, q, q, q, O, q, L)
        if dt == torch.float32:
            att = torch.randn(H, D, device="cuda")
            O, L = g.gatv2_attn_fwd(plan, ip, ix, q, q, att)
            g.gatv2_attn_bwd(plan, ip, ix, q, q, att, q, L)
    torch.cuda.synchronize()


def _dev(wl, nm):
    import torch
    if wl.dtype == "bf16":
        return torch.from_numpy(wl.bits[nm].view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(wl.feats[nm]).cuda()


def _library_bytes(fn):
    """Run fn and return (result, device bytes taken outside torch's allocator)."""
    import torch
    torch.cuda.synchronize()
    free0, _ = torch.cuda.mem_get_info()
    res0 = torch.cuda.memory_reserved()
    out = fn()
    torch.cuda.synchronize()
    free1, _ = torch.cuda.mem_get_info()
    res1 = torch.cuda.memory_reserved()
    return out, (free0 - free1) - (res1 - res0)


XSPLIT_MAX_RANGE = 12 << 20     # the header's bound on one eighth of the gathered tables


def _one_head_group(H, D, dtype):
    return H <= 64 // (D // (8 if dtype == "bf16" else 4))


def _ws_fwd(d, N, H, D, dtype="f32", gatv2=False):
    """Forward workspace: one partial (acc, m, l) per heavy group. The forward
    takes the source-range split groups when the plan has them, all heads fit
    one head group and one eighth of the gathered tables is at most 12 MiB
    (the rule the header states), else the plain groups."""
    size = 2 if dtype == "bf16" else 4
    gathered = N * H * D * size * (1 if gatv2 else 2)
    split = d["n_xsplit_groups"] > 0 and _one_head_group(H, D, dtype) and (gathered + 7) // 8 <= XSPLIT_MAX_RANGE
    return (d["n_xsplit_groups"] if split else d["n_groups"]) * (H * D + 2 * H) * 4


def _ws_bwd(d, N, H, D, gat, dtype="f32"):
    """Backward workspace: (LSE, Delta) per node and head, the destination
    pass's partials per heavy group, the source pass's per heavy source group,
    and for GATv2 the per-node d_att terms and their column-sum partials. The
    GATv2 destination pass takes the split groups under the forward's rule
    (gathered: the XS rows)."""
    rowlen = H * D
    size = 2 if dtype == "bf16" else 4
    na = d["n_groups"]
    if gat and _one_head_group(H, D, dtype) and d["n_xsplit_groups"] > 0 \
            and (N * rowlen * size + 7) // 8 <= XSPLIT_MAX_RANGE:
        na = d["n_xsplit_groups"]
    n = 2 * N * H + na * ((4 if gat else 2) * rowlen + H) + d["c_n_groups"] * 2 * rowlen
    if gat:
        n += N * rowlen + ((N + 63) // 64) * rowlen
    return n * 4


def _audit(g, plan, wl, E, name, fn, expect_ws):
    before = g.gnn_plan_export(plan)["workspace_bytes"]
    _, lib1 = _library_bytes(fn)
    d = g.gnn_plan_export(plan)
    grew = d["workspace_bytes"] - before
    say(f"  {name}: workspace {d['workspace_bytes'] / MIB:.2f} MiB (expected {expect_ws / MIB:.2f}), "
        f"library took {lib1 / MIB:.2f} MiB, E*H*2 = {2 * E * wl.heads / MIB:.1f} MiB")
    assert d["workspace_bytes"] == max(before, expect_ws), name
    assert d["largest_workspace_alloc"] < 2 * E * wl.heads, name
    assert lib1 <= max(grew, 0) + 2 * PAGE, (name, lib1, grew)
    _, lib2 = _library_bytes(fn)
    say(f"  {name} again: library took {lib2 / MIB:.2f} MiB, workspace "
        f"{g.gnn_plan_export(plan)['workspace_bytes'] / MIB:.2f} MiB")
    assert g.gnn_plan_export(plan)["workspace_bytes"] == d["workspace_bytes"], name
    assert lib2 <= PAGE, (name, "second call allocated", lib2)


@pytest.mark.parametrize("name,tiles", [("gatv2_zipf21_n100k", 0.0), ("gt_chunglu22_n2450k", 0.0),
                                        ("gt_comm16_n1m_deg27", 0.0), ("gt_comm16_n1m_deg27", 0.75)])
def test_memory_audit(g, name, tiles):
    import torch
    say("memory audit", name, "tiles" if tiles else "")
    backward = name != "gt_chunglu22_n2450k"
    wl = workloads.make(name, backward=backward)
    N, H, D = wl.n_nodes, wl.heads, wl.dim
    ip, ix = g.gnn_csr_build(torch.from_numpy(wl.src).cuda(), torch.from_numpy(wl.dst).cuda(), N)
    E = int(ix.numel())
    plan = g.gnn_plan_create(ip, ix, want_csc=backward, tile_density=tiles)
    d = g.gnn_plan_export(plan)
    say(f"  structure {d['structure_bytes'] / MIB:.1f} MiB for E = {E}")
    # buckets, CSC and launch orders are O(N + E) int32 arrays; tiles add O(#tiles) and a residual CSR
    assert d["structure_bytes"] <= 4 * (8 * (N + 1) + 3 * E) + 48 * d["n_tiles"] + 64 * MIB
    holder = {}
    if wl.kind == "gatv2":
        xd, xs, go = _dev(wl, "XD"), _dev(wl, "XS"), _dev(wl, "dO")
        att = torch.from_numpy(wl.att).cuda()

        def fwd():
            holder["fwd"] = g.gatv2_attn_fwd(plan, ip, ix, xd, xs, att)

        def bwd():
            holder["bwd"] = g.gatv2_attn_bwd(plan, ip, ix, xd, xs, att, go, holder["fwd"][1])
    else:
        q, k, v = _dev(wl, "Q"), _dev(wl, "K"), _dev(wl, "V")

        def fwd():
            holder["fwd"] = g.gnn_attn_fwd(plan, ip, ix, q, k, v)

        if backward:
            go = _dev(wl, "dO")

            def bwd():
                O, L = holder["fwd"]
                holder["bwd"] = g.gnn_attn_bwd(plan, ip, ix, q, k, v, O, go, L)
    _audit(g, plan, wl, E, "forward", fwd, _ws_fwd(d, N, H, D, wl.dtype, wl.kind == "gatv2"))
    if backward:
        _audit(g, plan, wl, E, "backward", bwd, _ws_bwd(d, N, H, D, wl.kind == "gatv2", wl.dtype))


def test_alloc_cap_fails_cleanly_midway(g, monkeypatch):
    """With GNN_ALLOC_CAP_BYTES between the sizes of a plan's allocations,
    gnn_plan_create fails with GNN_ERR_OOM part-way (after some arrays were
    allocated) and frees everything it took; a forward whose workspace would
    grow past the cap fails the same way and writes nothing; with the cap
    cleared both succeed."""
    import torch
    from io_aware_sparse_amd import GnnError
    wl = workloads.make("gatv2_zipf21_n100k", 20000, features=False)
    n = wl.n_nodes
    ip, ix = g.gnn_csr_build(torch.from_numpy(wl.src).cuda(), torch.from_numpy(wl.dst).cuda(), n)
    E = int(ix.numel())
    # the plan's first requests (validation, sortedness check, buckets) are far below
    # 16 * E bytes, the transposed adjacency's temporary (24 bytes per edge) above it
    monkeypatch.setenv("GNN_ALLOC_CAP_BYTES", str(16 * E))
    plans = []

    def attempt():
        try:
            plans.append(g.gnn_plan_create(ip, ix, want_csc=True, light_threshold=64, chunk=64))
        except GnnError as e:
            return e
    err, taken = _library_bytes(attempt)
    say(f"alloc cap {16 * E} B: {err}; library bytes left behind {taken}")
    assert err is not None and err.status == -4 and "GNN_ALLOC_CAP_BYTES" in str(err)
    assert not plans
    assert taken <= PAGE, taken
    monkeypatch.delenv("GNN_ALLOC_CAP_BYTES")
    plan = g.gnn_plan_create(ip, ix, want_csc=True, light_threshold=64, chunk=64)
    d = g.gnn_plan_export(plan)
    assert d["n_groups"] > 0 and d["workspace_bytes"] == 0
    H, D = 4, 32
    q = torch.randn(n, H, D, device="cuda")
    O = torch.full_like(q, 5.0)
    monkeypatch.setenv("GNN_ALLOC_CAP_BYTES", str(_ws_fwd(d, n, H, D) - 1))
    with pytest.raises(GnnError) as e:
        g.gnn_attn_fwd(plan, ip, ix, q, q, q, O=O)
    assert e.value.status == -4
    torch.cuda.synchronize()
    assert torch.all(O == 5.0) and g.gnn_plan_export(plan)["workspace_bytes"] == 0
    monkeypatch.setenv("GNN_ALLOC_CAP_BYTES", str(_ws_fwd(d, n, H, D)))
    g.gnn_attn_fwd(plan, ip, ix, q, q, q, O=O)
    torch.cuda.synchronize()
    assert g.gnn_plan_export(plan)["workspace_bytes"] == _ws_fwd(d, n, H, D)
    assert not torch.any(O == 5.0)
