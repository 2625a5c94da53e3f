"""GPU parity of the 16x16 MFMA tile path (bf16) against the fp64 oracle.

Tiled plans route rows of tiled row blocks (and sources of tiled column
blocks) through the matrix-core kernels, which also stream those rows'
residual edges; everything else stays on the CSR kernels. Graphs: the
community recipes at a few thousand nodes, and a graph with dense blocks of
varying fill plus hubs (ineligible blocks) and a ragged last block."""
import math

import numpy as np
import pytest

import oracle
import workloads
from _gpu import TOL, check, dev_feat, dev_i32, host, rand_feats, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def g():
    import io_aware_sparse_amd as g
    g.lib()
    return g


def _graph(g, kind):
    if kind == "blocks":
        rng = np.random.default_rng(400)
        n = 1000
        a = rng.random((n, n)) < 0.01
        for b0 in range(0, n - 15, 16):
            if rng.random() < 0.6:
                a[b0:b0 + 16, b0:b0 + 16] |= rng.random((16, 16)) < rng.uniform(0.6, 1.0)
            if rng.random() < 0.3:                   # dense off-diagonal blocks: several tiles per row
                c0 = 16 * int(rng.integers(1, n // 16))          # and per column block
                a[b0:b0 + 16, c0:c0 + 16] |= rng.random((16, 16)) < rng.uniform(0.6, 1.0)
        a[:, 7] = True
        a[333, :] = True
        dst, src = np.nonzero(a)
        src, dst = src.astype(np.int32), dst.astype(np.int32)
    else:
        wl = workloads.make(kind, 2048, features=False)
        src, dst, n = wl.src, wl.dst, wl.n_nodes
    rp, rx = oracle.csr_build(src, dst, n)
    ip, ix = g.gnn_csr_build(dev_i32(src), dev_i32(dst), n)
    assert np.array_equal(ip.cpu().numpy(), rp) and np.array_equal(ix.cpu().numpy(), rx)
    return ip, ix, rp, rx, n


def _check(name, x, ref, scale, dtype):
    check(name, x, ref, scale, dtype)


CASES = [(64, 8), (32, 16), (32, 4), (128, 2), (128, 5), (64, 3), (64, 1)]


@pytest.mark.parametrize("D,H", CASES)
@pytest.mark.parametrize("kind,tau,T", [("gt_comm16_n1m_deg27", 0.75, 512), ("gt_comm16_n1m_deg100", 0.75, 512),
                                        ("blocks", 0.5, 60)])
def test_tile_fwd_bwd_parity(g, D, H, kind, tau, T):
    say("tiles", kind, D, H, tau, T)
    ip, ix, rp, rx, n = _graph(g, kind)
    plan = g.gnn_plan_create(ip, ix, light_threshold=T, chunk=32, waves_per_group=4, tile_density=tau, want_csc=True)
    info = g.gnn_plan_export(plan)
    assert info["n_tiles"] > 0
    if kind == "blocks":                              # blocks with several tiles, both ways
        d = g.gnn_plan_export(plan, arrays=True)
        assert np.diff(d["tile_ptr"]).max() >= 2 and np.diff(d["ctile_ptr"]).max() >= 2
    rng = np.random.default_rng(D + 3 * H)
    Q, K, V, dO = rand_feats(rng, n, H, D, "bf16", k=4)
    q, k, v, go = (dev_feat(x, "bf16") for x in (Q, K, V, dO))
    O, L = g.gnn_attn_fwd(plan, ip, ix, q, k, v)
    dq, dk, dv = g.gnn_attn_bwd(plan, ip, ix, q, k, v, O, go, L)
    ref = oracle.gt_fwd(rp, rx, Q, K, V)
    _check("O", host(O), ref["O"], ref["SO"], "bf16")
    _check("LSE", host(L), ref["LSE"], ref["SL"], "f32")
    rb = oracle.gt_bwd(rp, rx, Q, K, V, dO)
    _check("dQ", host(dq), rb["dQ"], rb["SdQ"], "bf16")
    _check("dK", host(dk), rb["dK"], rb["SdK"], "bf16")
    _check("dV", host(dv), rb["dV"], rb["SdV"], "bf16")


def test_tile_plan_with_fp32_uses_csr_path(g):
    ip, ix, rp, rx, n = _graph(g, "gt_comm16_n1m_deg27")
    plan = g.gnn_plan_create(ip, ix, tile_density=0.75, want_csc=True)
    rng = np.random.default_rng(5)
    Q, K, V, dO = rand_feats(rng, n, 4, 32, "f32", k=4)
    q, k, v, go = (dev_feat(x, "f32") for x in (Q, K, V, dO))
    O, L = g.gnn_attn_fwd(plan, ip, ix, q, k, v)
    dq, dk, dv = g.gnn_attn_bwd(plan, ip, ix, q, k, v, O, go, L)
    ref = oracle.gt_fwd(rp, rx, Q, K, V)
    rb = oracle.gt_bwd(rp, rx, Q, K, V, dO)
    _check("O", host(O), ref["O"], ref["SO"], "f32")
    _check("dK", host(dk), rb["dK"], rb["SdK"], "f32")


def test_tile_path_deterministic_and_close_to_csr_path(g):
    import torch
    ip, ix, rp, rx, n = _graph(g, "gt_comm16_n1m_deg27")
    tiled = g.gnn_plan_create(ip, ix, tile_density=0.75, want_csc=True)
    plain = g.gnn_plan_create(ip, ix, want_csc=True)
    rng = np.random.default_rng(6)
    q, k, v, go = (dev_feat(x, "bf16") for x in rand_feats(rng, n, 8, 64, "bf16", k=4))
    runs = []
    for plan in (tiled, tiled, plain):
        O, L = g.gnn_attn_fwd(plan, ip, ix, q, k, v)
        dq, dk, dv = g.gnn_attn_bwd(plan, ip, ix, q, k, v, O, go, L)
        runs.append([t.clone() for t in (O, L, dq, dk, dv)])
    for a, b in zip(runs[0], runs[1]):
        assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a,
                           b.view(torch.int16) if b.dtype == torch.bfloat16 else b)
    for a, b in zip(runs[0], runs[2]):
        d = (a.float() - b.float()).abs().max().item()
        assert d < 5e-2 * max(1.0, b.float().abs().max().item()), d
