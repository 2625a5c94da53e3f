"""The allocation-free Graph-Transformer forward (gnn_attn_fwd_noalloc)
against gnn_attn_fwd, both through the C ABI.

Two calls in a row, the second on a smaller graph (and another dtype and head
shape), each with heavy rows whose partial states go to the fixed scratch:
outputs bitwise equal to gnn_attn_fwd's on an identical plan and within the
oracle's bar; the plan's workspace never grows and device free memory does
not change across a call. Also a tiled plan, the scratch-size error (nothing
launched), the timing guard, and the call recorded into a HIP graph whose
replays (eager work on the shared scratch in between) equal the eager call."""
import numpy as np
import pytest

import oracle
import workloads
from _gpu import check, dev_i32, host, rand_feats, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def g():
    import io_aware_sparse_amd as g
    g.lib()
    return g


def _graph(name, n):
    wl = workloads.make(name, n, features=False)
    rp, rx = oracle.csr_build(wl.src, wl.dst, n)
    return rp, rx


def _run_pair(g, rp, rx, dtype, H, D, seed, opts):
    """noalloc on one plan, gnn_attn_fwd on an identical second plan."""
    import torch
    n = rp.size - 1
    ip, ix = dev_i32(rp), dev_i32(rx)
    plan_a = g.gnn_plan_create(ip, ix, **opts)
    plan_b = g.gnn_plan_create(ip, ix, **opts)
    info = g.gnn_plan_export(plan_a)
    Qh, Kh, Vh = rand_feats(np.random.default_rng(seed), n, H, D, dtype)
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    q, k, v = (torch.from_numpy(x).cuda().to(tdt) for x in (Qh, Kh, Vh))
    O = torch.full_like(q, 7.0)
    L = torch.full((n, H), 7.0, dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    g.gnn_attn_fwd_noalloc(plan_a, ip, ix, q, k, v, O, L)
    torch.cuda.synchronize()
    Or, Lr = g.gnn_attn_fwd(plan_b, ip, ix, q, k, v)
    torch.cuda.synchronize()
    return plan_a, info, (ip, ix, q, k, v), (Qh, Kh, Vh), (O, L), (Or, Lr)


def _compare(g, name, rp, rx, dtype, H, D, seed, opts, need_heavy=True):
    import torch
    plan_a, info, dev, hostf, (O, L), (Or, Lr) = _run_pair(g, rp, rx, dtype, H, D, seed, opts)
    say(f"noalloc {name}: N={rp.size - 1} E={rx.size} {dtype} H={H} D={D} heavy groups {info['n_groups']} "
        f"tiles {info['n_tiles']}")
    if need_heavy:
        assert info["n_groups"] > 0, "case must exercise the scratch"
    assert torch.equal(O.view(torch.int16) if O.dtype == torch.bfloat16 else O.view(torch.int32),
                       Or.view(torch.int16) if Or.dtype == torch.bfloat16 else Or.view(torch.int32)), "O differs"
    assert torch.equal(L.view(torch.int32), Lr.view(torch.int32)), "LSE differs"
    ref = oracle.gt_fwd(rp, rx, *hostf)
    check(f"{name} O", host(O), ref["O"], ref["SO"], dtype)
    check(f"{name} LSE", host(L), ref["LSE"], ref["SL"], "f32")
    assert g.gnn_plan_export(plan_a)["workspace_bytes"] == 0, "plan workspace grew"
    return plan_a, dev, O, L


def test_noalloc_matches_gnn_attn_fwd_twice(g):
    import torch
    # first call: 6,000-node power-law graph, fp32, H = 4, D = 32, heavy rows (T = 24, C = 16, W = 4)
    rp, rx = _graph("gt_chunglu25_n169k", 6000)
    opts = dict(light_threshold=24, chunk=16, waves_per_group=4)
    plan1, dev1, O1, L1 = _compare(g, "call 1", rp, rx, "f32", 4, 32, 11, opts)
    # second call, smaller: 1,500-node Zipf graph, bf16, H = 2, D = 64
    rp2, rx2 = _graph("gatv2_zipf21_n100k", 1500)
    _compare(g, "call 2 (smaller)", rp2, rx2, "bf16", 2, 64, 12, opts)
    # the same first problem again after the smaller one: the scratch keeps the
    # last call's contents, and the result must not depend on them
    ip, ix, q, k, v = dev1
    O = torch.empty_like(q)
    L = torch.empty(L1.shape, dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    free0 = torch.cuda.mem_get_info()[0]
    g.gnn_attn_fwd_noalloc(plan1, ip, ix, q, k, v, O, L)
    torch.cuda.synchronize()
    free1 = torch.cuda.mem_get_info()[0]
    say(f"  device free memory across a call: {free0} -> {free1}")
    assert free1 == free0, "device memory changed across the call"
    assert torch.equal(O.view(torch.int32), O1.view(torch.int32)) and torch.equal(L.view(torch.int32),
                                                                                 L1.view(torch.int32))


def test_noalloc_tiled_plan(g):
    rp, rx = _graph("gt_comm16_n1m_deg27", 2048)
    _compare(g, "tiled", rp, rx, "bf16", 8, 64, 13, dict(tile_density=0.75), need_heavy=False)


def test_noalloc_scratch_limit_and_timing_guard(g):
    import torch
    import io_aware_sparse_amd as gg
    # every row heavy and every entry its own group: n_groups * (H*D + 2H) * 4 > 16 MiB
    rng = np.random.default_rng(5)
    n, H, D = 1000, 8, 128
    src = rng.integers(0, n, 6000).astype(np.int32)
    dst = rng.integers(0, n, 6000).astype(np.int32)
    rp, rx = oracle.csr_build(src, dst, n)
    ip, ix = dev_i32(rp), dev_i32(rx)
    plan = g.gnn_plan_create(ip, ix, light_threshold=0, chunk=1, waves_per_group=1)
    groups = g.gnn_plan_export(plan)["n_groups"]
    need = groups * (H * D + 2 * H) * 4
    assert need > (16 << 20)
    q = torch.randn(n, H, D, device="cuda")
    O = torch.full_like(q, 3.0)
    with pytest.raises(gg.GnnError) as e:
        g.gnn_attn_fwd_noalloc(plan, ip, ix, q, q, q, O)
    assert e.value.status == -7
    torch.cuda.synchronize()
    assert torch.all(O == 3.0), "a rejected call launched work"
    say(f"noalloc: {groups} groups need {need} bytes -> GNN_ERR_SCRATCH")
    # the same call fits with a coarser plan
    plan2 = g.gnn_plan_create(ip, ix, light_threshold=0, chunk=4, waves_per_group=1)
    g.gnn_attn_fwd_noalloc(plan2, ip, ix, q, q, q, O)
    Or, _ = g.gnn_attn_fwd(plan2, ip, ix, q, q, q)
    torch.cuda.synchronize()
    assert torch.equal(O, Or)
    # per-kernel timing on the plan is refused (event records are not allocation-free)
    g.gnn_plan_set_timing(plan2, True)
    with pytest.raises(gg.GnnError) as e:
        g.gnn_attn_fwd_noalloc(plan2, ip, ix, q, q, q, O)
    assert e.value.status == -2
    g.gnn_plan_set_timing(plan2, False)


def test_noalloc_under_graph_capture(g):
    """The allocation-free forward recorded into a HIP graph and replayed: each
    replay, after eager work that overwrites the outputs and the shared scratch
    (another allocation-free call on another graph with heavy rows), equals the
    eager result bit for bit."""
    import torch
    if g.gnn_build_checked():
        pytest.skip("the checked build reads its index-check flags after every call (a synchronising copy), "
                    "which a capturing stream does not allow")
    rp, rx = _graph("gt_chunglu25_n169k", 6000)
    rp2, rx2 = _graph("gatv2_zipf21_n100k", 1500)
    n, n2, H, D = rp.size - 1, rp2.size - 1, 4, 32
    ip, ix, ip2, ix2 = dev_i32(rp), dev_i32(rx), dev_i32(rp2), dev_i32(rx2)
    opts = dict(light_threshold=24, chunk=16, waves_per_group=4)
    plan, plan2 = g.gnn_plan_create(ip, ix, **opts), g.gnn_plan_create(ip2, ix2, **opts)
    assert g.gnn_plan_export(plan)["n_groups"] > 0 and g.gnn_plan_export(plan2)["n_groups"] > 0
    q, k, v = (torch.from_numpy(x).cuda() for x in rand_feats(np.random.default_rng(21), n, H, D, "f32"))
    q2, k2, v2 = (torch.from_numpy(x).cuda() for x in rand_feats(np.random.default_rng(22), n2, H, D, "f32"))
    O_ref, L_ref = torch.empty_like(q), torch.empty((n, H), device="cuda")
    g.gnn_attn_fwd_noalloc(plan, ip, ix, q, k, v, O_ref, L_ref)          # eager reference
    O, L = torch.empty_like(q), torch.empty((n, H), device="cuda")
    O2, L2 = torch.empty_like(q2), torch.empty((n2, H), device="cuda")
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        g.gnn_attn_fwd_noalloc(plan, ip, ix, q, k, v, O, L)             # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=s):
        g.gnn_attn_fwd_noalloc(plan, ip, ix, q, k, v, O, L)
    torch.cuda.synchronize()
    for r in range(4):
        O.fill_(7.0)
        L.fill_(7.0)
        g.gnn_attn_fwd_noalloc(plan2, ip2, ix2, q2, k2, v2, O2, L2)      # eager work on the shared scratch
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(O.view(torch.int32), O_ref.view(torch.int32)), f"replay {r}: O differs"
        assert torch.equal(L.view(torch.int32), L_ref.view(torch.int32)), f"replay {r}: LSE differs"
    say("noalloc: graph capture, 4 replays bitwise equal to the eager call")
