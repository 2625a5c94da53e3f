"""Child process of tests/test_gpu_checked.py: runs the checked build of the
library (GNN_CHECKED=1 in its environment) on a good graph, saving every
output, and on graphs with an index outside [0, N), printing the statuses.
It confirms that the checked build is the one loaded before it passes a bad
index to any kernel, and exits otherwise."""
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

H, D, F = 4, 32, 64


def make_case():
    """A seeded graph (hubs on the heavy path for the small threshold used) and
    its feature tables, as numpy arrays."""
    rng = np.random.default_rng(77)
    n = 3000
    deg = rng.poisson(6, n)
    deg[rng.choice(n, 20, replace=False)] = rng.integers(100, 400, 20)
    ix = np.concatenate([np.sort(rng.integers(0, n, d)) for d in deg]).astype(np.int32)
    ip = np.concatenate([[0], np.cumsum(deg)]).astype(np.int32)
    feats = {k: rng.standard_normal((n, H, D)).astype(np.float32) for k in ("Q", "K", "V", "dO")}
    feats["X"] = rng.standard_normal((n, F)).astype(np.float32)
    feats["att"] = rng.standard_normal((H, D)).astype(np.float32)
    return ip, ix, feats


def run_all(g, ip, ix, feats):
    """Every kernel family on a plan (and the plan-less forward): host arrays."""
    import torch
    dev = {k: torch.from_numpy(v).cuda() for k, v in feats.items()}
    ipd, ixd = torch.from_numpy(ip).cuda(), torch.from_numpy(ix).cuda()
    plan = g.gnn_plan_create(ipd, ixd, light_threshold=64, chunk=32, want_csc=True)
    out = {}
    out["O"], out["LSE"] = g.gnn_attn_fwd(plan, ipd, ixd, dev["Q"], dev["K"], dev["V"])
    out["dQ"], out["dK"], out["dV"] = g.gnn_attn_bwd(plan, ipd, ixd, dev["Q"], dev["K"], dev["V"], out["O"],
                                                     dev["dO"], out["LSE"])
    out["O_noplan"], _ = g.gnn_attn_fwd(None, ipd, ixd, dev["Q"], dev["K"], dev["V"])
    out["gO"], out["gLSE"] = g.gatv2_attn_fwd(plan, ipd, ixd, dev["Q"], dev["K"], dev["att"])
    dxd, dxs, _, da = g.gatv2_attn_bwd(plan, ipd, ixd, dev["Q"], dev["K"], dev["att"], dev["dO"], out["gLSE"])
    out["dXD"], out["dXS"], out["d_att"] = dxd, dxs, da
    out["max"], out["arg"] = g.gnn_reduce_fwd(plan, ipd, ixd, dev["X"])
    out["max_grad"] = g.gnn_reduce_bwd(plan, ipd, ixd, dev["X"], out["arg"])
    g.gnn_spmm_prepare(plan, "gcn")
    out["Y"] = g.gnn_spmm(plan, ipd, ixd, dev["X"])
    out["YT"] = g.gnn_spmm(plan, ipd, ixd, dev["X"], transpose=True)
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in out.items()}


def status_of(g, fn):
    try:
        fn()
        return 0
    except g.GnnError as e:
        return e.status


def main(outdir):
    import torch
    import io_aware_sparse_amd as g
    if not g.gnn_build_checked():
        print(json.dumps({"checked": False}), flush=True)
        return 3
    ip, ix, feats = make_case()
    np.savez(os.path.join(outdir, "checked.npz"), **run_all(g, ip, ix, feats))
    n = ip.size - 1
    Q, K, V = (torch.from_numpy(feats[k]).cuda() for k in ("Q", "K", "V"))
    ipd = torch.from_numpy(ip).cuda()
    good = torch.from_numpy(ix).cuda()
    bad = ix.copy()
    bad[5], bad[ip[100] + 1] = n + 5, -3          # out of range in a short row and below zero in another
    badd = torch.from_numpy(bad).cuda()
    O = torch.empty_like(Q)
    res = {"checked": True}
    # validated entry points: the graph check rejects the call before any compute kernel
    res["fwd_noplan"] = status_of(g, lambda: g.gnn_attn_fwd(None, ipd, badd, Q, K, V))
    # a plan built on good arrays that the caller changed afterwards
    mut = good.clone()
    plan = g.gnn_plan_create(ipd, mut)
    mut[5] = n + 5
    res["fwd_plan_arrays_changed"] = status_of(g, lambda: g.gnn_attn_fwd(plan, ipd, mut, Q, K, V))
    # the allocation-free forward skips the graph check: its kernels meet the bad index, check it and report it
    res["noalloc_noplan"] = status_of(g, lambda: g.gnn_attn_fwd_noalloc(None, ipd, badd, Q, K, V, O))
    res["noalloc_plan_arrays_changed"] = status_of(g, lambda: g.gnn_attn_fwd_noalloc(plan, ipd, mut, Q, K, V, O))
    # the same plan-less call on the good graph afterwards: the flags were cleared
    res["noalloc_after"] = status_of(g, lambda: g.gnn_attn_fwd_noalloc(None, ipd, good, Q, K, V, O))
    torch.cuda.synchronize()
    np.save(os.path.join(outdir, "O_after.npy"), O.cpu().numpy())
    print(json.dumps(res), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main(sys.argv[1]))
