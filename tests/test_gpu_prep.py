"""GPU preprocessor parity: CSR build, degree bucketing and the transposed
adjacency must equal the oracle's integer definitions bit for bit."""
import numpy as np
import pytest

import oracle
import workloads
from _gpu import dev_i32, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def g():
    import io_aware_sparse_amd as g
    g.lib()
    return g


def _csr_case(g, src, dst, n, self_loops):
    say("csr_build", n, src.size, self_loops)
    ip, ix = g.gnn_csr_build(dev_i32(src), dev_i32(dst), n, add_self_loops=self_loops)
    rp, rx = oracle.csr_build(src, dst, n, add_self_loops=self_loops)
    assert np.array_equal(ip.cpu().numpy(), rp)
    assert np.array_equal(ix.cpu().numpy(), rx)
    return ip, ix, rp, rx


@pytest.mark.parametrize("seed,n,m", [(0, 1, 0), (1, 1, 5), (2, 2, 7), (3, 37, 300), (4, 1000, 20000),
                                      (5, 5000, 4097), (6, 70000, 300000)])
@pytest.mark.parametrize("self_loops", [True, False])
def test_csr_build_random(g, seed, n, m, self_loops):
    rng = np.random.default_rng(seed)
    src = rng.integers(0, n, m).astype(np.int32)
    dst = rng.integers(0, n, m).astype(np.int32)
    if m > 10:
        dup = rng.integers(0, m, m // 5)          # explicit duplicates and self-pairs
        src[dup[: dup.size // 2]] = dst[dup[: dup.size // 2]]
        src = np.concatenate([src, src[dup]])
        dst = np.concatenate([dst, dst[dup]])
    _csr_case(g, src, dst, n, self_loops)


@pytest.mark.parametrize("name,n", [("gt_uniform_n2708", None), ("gt_chunglu25_n169k", 20000),
                                    ("gatv2_zipf21_n100k", 20000), ("gt_comm16_n1m_deg100", 4096)])
def test_csr_build_workloads(g, name, n):
    wl = workloads.make(name, n, features=False)
    _csr_case(g, wl.src, wl.dst, wl.n_nodes, True)


def test_csr_build_rejects_bad_endpoint(g):
    src = np.array([0, 1, 7], np.int32)
    dst = np.array([1, 2, 0], np.int32)
    with pytest.raises(g.GnnError) as e:
        g.gnn_csr_build(dev_i32(src), dev_i32(dst), 5)
    assert e.value.status == -6


@pytest.mark.parametrize("order", [0, 1, 2])
@pytest.mark.parametrize("T,C,W", [(0, 1, 1), (0, 5, 4), (3, 2, 2), (16, 8, 2), (64, 64, 8), (512, 512, 4),
                                   (10 ** 9, 512, 4)])
def test_buckets_and_csc(g, T, C, W, order):
    wl = workloads.make("gatv2_zipf21_n100k", 12000, features=False)
    n = wl.n_nodes
    ip, ix, rp, rx = _csr_case(g, wl.src, wl.dst, n, True)
    say("plan", T, C, W)
    plan = g.gnn_plan_create(ip, ix, light_threshold=T, chunk=C, waves_per_group=W, want_csc=True,
                             sched_order=order)
    d = g.gnn_plan_export(plan, arrays=True)
    ref = oracle.bucketing(rp, T, C, W)
    for k in ("light", "heavy", "groups", "partial_ofs"):
        assert np.array_equal(d[k], ref[k]), k
    assert np.array_equal(d["light_sched"], oracle.launch_order(rp, ref["light"], order, T))
    assert np.array_equal(d["light_by_degree"], oracle.launch_order(rp, ref["light"], 3, T))
    cip, cix = oracle.csc(rp, rx, n)
    assert np.array_equal(d["cindptr"], cip) and np.array_equal(d["cindices"], cix)
    cref = oracle.bucketing(cip, T, C, W)
    for k in ("light", "heavy", "groups", "partial_ofs"):
        assert np.array_equal(d["c_" + k], cref[k]), "c_" + k
    assert np.array_equal(d["c_light_sched"], oracle.launch_order(cip, cref["light"], order, T))
    # the long light rows (a wave each in the packed launches) head the packed order
    assert d["n_long_light"] == int((np.diff(rp)[ref["light"]] > 128).sum())
    assert d["c_n_long_light"] == int((np.diff(cip)[cref["light"]] > 128).sum())
    assert np.array_equal(d["c_light_by_degree"], oracle.launch_order(cip, cref["light"], 3, T))
    assert d["n_light"] + d["n_heavy"] == n
    # the source-range split of the heavy rows (built by default on sorted rows)
    if ref["heavy"].size:
        xref = oracle.xsplit(rp, rx, ref["heavy"], n, C)
        for k in ("groups", "partial_ofs", "order"):
            assert np.array_equal(d["xsplit_" + k], xref[k]), "xsplit_" + k
    else:
        assert d["n_xsplit_groups"] == 0


@pytest.mark.parametrize("name,n", [("gt_chunglu25_n169k", 20000), ("gt_comm16_n1m_deg100", 4096),
                                    ("gatv2_zipf21_n100k", 100000)])
def test_xsplit(g, name, n):
    """The source-range split bit for bit against the oracle on other graph
    shapes (the full-size Zipf graph among them); none without the option or
    on rows that are not sorted."""
    wl = workloads.make(name, n, features=False)
    n = wl.n_nodes
    ip, ix, rp, rx = _csr_case(g, wl.src, wl.dst, n, True)
    for T, C, W in ((512, 512, 4), (16, 8, 2)):
        d = g.gnn_plan_export(g.gnn_plan_create(ip, ix, light_threshold=T, chunk=C, waves_per_group=W), arrays=True)
        heavy = oracle.bucketing(rp, T, C, W)["heavy"]
        say(f"xsplit {name} T={T}: {d['n_xsplit_groups']} groups for {heavy.size} heavy rows, "
            f"{d['n_xsplit_slots']} slots")
        if heavy.size == 0:
            assert d["n_xsplit_groups"] == 0
        else:
            xref = oracle.xsplit(rp, rx, heavy, n, C)
            for k in ("groups", "partial_ofs", "order"):
                assert np.array_equal(d["xsplit_" + k], xref[k]), ("xsplit_" + k, T)
        off = g.gnn_plan_export(g.gnn_plan_create(ip, ix, light_threshold=T, chunk=C, waves_per_group=W,
                                                  xcd_split=False))
        assert off["n_xsplit_groups"] == 0 and off["n_xsplit_slots"] == 0
    # rows not sorted: the plan keeps the plain groups only
    rx2 = rx.copy()
    big = int(np.argmax(np.diff(rp)))
    rx2[rp[big]:rp[big + 1]] = rx2[rp[big]:rp[big + 1]][::-1]
    d = g.gnn_plan_export(g.gnn_plan_create(ip, dev_i32(rx2)))
    assert d["rows_sorted"] == 0 and d["n_xsplit_groups"] == 0


def test_plan_rejects_inconsistent_graph(g):
    import torch
    ip = dev_i32(np.array([0, 2, 3], np.int32))
    ix = dev_i32(np.array([0, 1, 1, 0], np.int32))       # indptr[N] = 3 != E = 4
    with pytest.raises(g.GnnError) as e:
        g.gnn_plan_create(ip, ix)
    assert e.value.status == -6
    ix = dev_i32(np.array([0, 5, 1], np.int32))          # index out of range
    with pytest.raises(g.GnnError) as e:
        g.gnn_plan_create(ip, ix)
    assert e.value.status == -6
    torch.cuda.synchronize()


def test_library_loaded_before_torch_in_fresh_process():
    """Loading the library before anything else imported torch must still
    leave one HIP runtime in the process (regression: allocations failed)."""
    import os
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    code = ("import io_aware_sparse_amd as g; g.lib(); import torch; "
            "s = torch.arange(10, dtype=torch.int32).cuda(); d = torch.roll(s, 1).contiguous(); "
            "ip, ix = g.gnn_csr_build(s, d, 10); assert ip.cpu().tolist()[-1] == 20; print('ok')")
    r = subprocess.run([sys.executable, "-c", code], cwd=root, capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and r.stdout.strip().endswith("ok"), r.stdout + r.stderr


def _tile_graphs():
    rng = np.random.default_rng(300)
    out = []
    for name in ("gt_comm16_n1m_deg100", "gt_comm16_n1m_deg27"):
        wl = workloads.make(name, 4096, features=False)
        out.append((name, wl.src, wl.dst, wl.n_nodes))
    n = 1000                                   # dense blocks of varying fill + hubs + ragged last block
    a = rng.random((n, n)) < 0.01
    for b0 in range(0, n - 15, 16):
        if rng.random() < 0.6:
            a[b0:b0 + 16, b0:b0 + 16] |= rng.random((16, 16)) < rng.uniform(0.5, 1.0)
    a[:, 7] = True                             # a source of out-degree n
    a[333, :] = True                           # a row of in-degree n
    dst, src = np.nonzero(a)
    out.append(("blocks+hubs", src.astype(np.int32), dst.astype(np.int32), n))
    return out


@pytest.mark.parametrize("case", range(3))
@pytest.mark.parametrize("tau,T", [(0.75, 512), (0.5, 40), (1.0, 10 ** 6), (0.1, 512)])
def test_tile_census(g, case, tau, T):
    name, src, dst, n = _tile_graphs()[case]
    ip, ix, rp, rx = _csr_case(g, src, dst, n, True)
    say("tiles", name, tau, T)
    plan = g.gnn_plan_create(ip, ix, light_threshold=T, chunk=64, waves_per_group=4, tile_density=tau, want_csc=True)
    d = g.gnn_plan_export(plan, arrays=True)
    import math
    ref = oracle.tile_census(rp, rx, n, max(1, math.ceil(tau * 256 - 1e-9)), T)
    assert d["n_tiles"] == ref["tile_rc"].shape[0]
    for k in ("tile_rc", "tile_mask", "tile_ptr", "trb", "rindptr", "rindices", "light_nt", "ctile", "tcb",
              "rcindptr", "rcindices", "c_light_nt"):
        assert np.array_equal(d[k], np.asarray(ref[k]).reshape(d[k].shape)), k
    n_pop = int(sum(bin(int(w)).count("1") for w in d["tile_mask"].ravel()))
    assert n_pop + d["n_residual"] == rx.size
    say(f"  tiles {d['n_tiles']} residual {d['n_residual']} of {rx.size}")


def _bits(t):
    return t.contiguous().view(-1).view(__import__("torch").uint8).cpu()


@pytest.mark.parametrize("dtype,H,D,F", [("f32", 4, 64, 256), ("bf16", 8, 64, 512)])
def test_results_do_not_depend_on_launch_order(g, dtype, H, D, F):
    """The launch order of the light list only schedules work: each light row
    is computed by one wave on its own, so every output of every kernel family
    (GT forward and backward, GATv2 forward and backward, the max reduction and
    its gradient, both SpMM products) is bit for bit the same under launch
    orders 0, 1 and 2. Rows of 1 KiB run one per wave, from the launch order;
    a small threshold and chunk put hubs on the heavy path as well."""
    import torch
    wl = workloads.make("gatv2_zipf21_n100k", 12000, features=False)
    n = wl.n_nodes
    ip, ix, rp, rx = _csr_case(g, wl.src, wl.dst, n, True)
    gen = torch.Generator(device="cpu").manual_seed(5)
    dt = torch.float32 if dtype == "f32" else torch.bfloat16
    rnd = lambda *shape: torch.randn(*shape, generator=gen).to(dt).cuda()
    Q, K, V, dO = rnd(n, H, D), rnd(n, H, D), rnd(n, H, D), rnd(n, H, D)
    att = torch.randn(H, D, generator=gen).cuda()
    X, dY = rnd(n, F), rnd(n, F)
    outs = []
    for order in (0, 1, 2):
        say("launch order", order, dtype, H, D, F)
        plan = g.gnn_plan_create(ip, ix, light_threshold=96, chunk=64, want_csc=True, sched_order=order)
        O, LSE = g.gnn_attn_fwd(plan, ip, ix, Q, K, V)
        r = [O, LSE, *g.gnn_attn_bwd(plan, ip, ix, Q, K, V, O, dO, LSE)]
        GO, GL = g.gatv2_attn_fwd(plan, ip, ix, Q, K, att)
        r += [GO, GL] + [t for t in g.gatv2_attn_bwd(plan, ip, ix, Q, K, att, dO, GL) if t is not None]
        R, arg = g.gnn_reduce_fwd(plan, ip, ix, X)
        r += [R, arg, g.gnn_reduce_bwd(plan, ip, ix, dY, arg)]
        g.gnn_spmm_prepare(plan, "gcn")
        r += [g.gnn_spmm(plan, ip, ix, X), g.gnn_spmm(plan, ip, ix, X, transpose=True)]
        torch.cuda.synchronize()
        outs.append([_bits(t) for t in r])
    names = ["O", "LSE", "dQ", "dK", "dV", "gatv2 O", "gatv2 LSE", "dXD", "dXS", "d_att", "max", "argmax",
             "max grad", "spmm", "spmm transposed"]
    assert len(outs[0]) == len(names)
    for order, o in ((1, outs[1]), (2, outs[2])):
        for nm, a, b in zip(names, outs[0], o):
            assert torch.equal(a, b), f"{nm} differs between launch orders 0 and {order}"
