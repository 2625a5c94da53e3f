"""Concurrent use of the library from two host threads on two streams.

Each thread owns a plan and a stream (default priority) and runs the GT
forward, the LSE-recompute backward and the SpMM with its transpose several
times, while the other thread does the same on another graph (or, in the
second case, on the same graph with its own plan). The calls release the
interpreter lock, so the host code and the kernels of both threads overlap.
A plan's workspace and scratch belong to it and the kernels are
deterministic, so every output must equal, bit for bit, the same call run
alone on the default stream; one set is also checked against the oracle."""
import threading

import numpy as np
import pytest

import oracle
import workloads
from _gpu import check, dev_i32, say

pytestmark = pytest.mark.gpu

ITERS = 6


@pytest.fixture(scope="module")
def g():
    import io_aware_sparse_amd as g
    g.lib()
    return g


def _case(g, name, n, H, D, dtype, seed):
    import torch
    wl = workloads.make(name, n, features=False)
    rp, rx = oracle.csr_build(wl.src, wl.dst, n)
    ip, ix = g.gnn_csr_build(dev_i32(wl.src), dev_i32(wl.dst), n)
    plan = g.gnn_plan_create(ip, ix, want_csc=True)
    g.gnn_spmm_prepare(plan, "gcn")
    gen = torch.Generator(device="cuda").manual_seed(seed)
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    q, k, v, go = (torch.randn((n, H, D), generator=gen, device="cuda", dtype=tdt) for _ in range(4))
    return dict(rp=rp, rx=rx, ip=ip, ix=ix, plan=plan, q=q, k=k, v=v, go=go, X=q.view(n, H * D),
                dY=go.view(n, H * D), n=n, H=H, D=D, dtype=dtype)


def _outputs(c):
    import torch
    n, H, D = c["n"], c["H"], c["D"]
    e = lambda: torch.empty_like(c["q"])                                         # noqa: E731
    return dict(O=e(), L=torch.empty((n, H), dtype=torch.float32, device="cuda"), dQ=e(), dK=e(), dV=e(),
                Y=torch.empty_like(c["X"]), YT=torch.empty_like(c["X"]))


def _run(g, c, out, stream, iters):
    a = (c["plan"], c["ip"], c["ix"])
    for _ in range(iters):
        g.gnn_attn_fwd(*a, c["q"], c["k"], c["v"], O=out["O"], LSE=out["L"], stream=stream)
        g.gnn_attn_bwd(*a, c["q"], c["k"], c["v"], out["O"], c["go"], out["L"], dQ=out["dQ"], dK=out["dK"],
                       dV=out["dV"], stream=stream)
        g.gnn_spmm(*a, c["X"], Y=out["Y"], stream=stream)
        g.gnn_spmm(*a, c["dY"], transpose=True, Y=out["YT"], stream=stream)


def _concurrent(g, cases):
    """Run every case in its own thread and stream; returns their outputs."""
    import torch
    outs = [_outputs(c) for c in cases]
    streams = [torch.cuda.Stream() for _ in cases]
    for s in streams:
        s.wait_stream(torch.cuda.current_stream())
    errors = []

    def work(i):
        try:
            with torch.cuda.stream(streams[i]):
                _run(g, cases[i], outs[i], streams[i], ITERS)
        except Exception as ex:                                                  # re-raised below
            errors.append(ex)

    threads = [threading.Thread(target=work, args=(i,)) for i in range(len(cases))]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    torch.cuda.synchronize()
    if errors:
        raise errors[0]
    return outs


def _same(a, b):
    import torch
    return all(torch.equal(a[k].view(torch.int16) if a[k].dtype == torch.bfloat16 else a[k].view(torch.int32),
                           b[k].view(torch.int16) if b[k].dtype == torch.bfloat16 else b[k].view(torch.int32))
               for k in a)


@pytest.mark.parametrize("same_graph", [False, True])
def test_two_threads_two_streams(g, same_graph):
    import torch
    A = _case(g, "gt_chunglu25_n169k", 40_000, 4, 32, "f32", 1)
    B = _case(g, "gt_chunglu25_n169k", 40_000, 4, 32, "f32", 2) if same_graph else \
        _case(g, "gt_comm16_n1m_deg27", 60_000, 8, 64, "bf16", 2)
    say(f"two threads, two streams: {A['rx'].size} and {B['rx'].size} entries, "
        f"{'same graph, separate plans' if same_graph else 'two graphs'}, {ITERS} rounds each")
    alone = []
    for c in (A, B):
        out = _outputs(c)
        _run(g, c, out, torch.cuda.current_stream(), 1)
        alone.append(out)
    torch.cuda.synchronize()
    together = _concurrent(g, [A, B])
    for name, x, y in (("A", alone[0], together[0]), ("B", alone[1], together[1])):
        ok = _same(x, y)
        say(f"  {name}: concurrent outputs equal the lone call bit for bit: {ok}")
        assert ok, name
    rows = np.random.default_rng(5).choice(A["n"], 500, replace=False)
    Q, K, V = (A[t].cpu().numpy() for t in ("q", "k", "v"))
    ref = oracle.gt_fwd(A["rp"], A["rx"], Q, K, V, rows=rows)
    idx = torch.from_numpy(rows).cuda()
    check("O (A, concurrent)", together[0]["O"].index_select(0, idx).double().cpu().numpy(), ref["O"], ref["SO"],
          "f32")
