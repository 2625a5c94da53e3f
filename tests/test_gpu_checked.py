"""The checked build (GNN_CHECKED): on good graphs every output equals the
normal build's bit for bit; a graph index outside [0, N) makes the call
return GNN_ERR_BAD_GRAPH, from the graph check of the validated entry points
or, in the allocation-free forward (which skips that check), from the
kernels' own index checks, which replace the index by row 0 so that no access
leaves the tables. The checked library runs in a child process that confirms
it is loaded before it passes a bad index to any kernel."""
import json
import os
import subprocess
import sys

import numpy as np
import pytest

from _gpu import say

pytestmark = pytest.mark.gpu
HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.fixture(scope="module")
def g():
    import io_aware_sparse_amd as g
    g.lib()
    return g


def test_checked_build(g, tmp_path):
    import _checked_child as child
    lib = os.path.join(os.path.dirname(g.LIB_PATH), "libgnn_attn_checked.so")
    if not os.path.exists(lib):
        pytest.fail(f"checked build missing: {lib}")
    assert not g.gnn_build_checked()
    env = dict(os.environ, GNN_CHECKED="1")
    r = subprocess.run([sys.executable, "-u", os.path.join(HERE, "_checked_child.py"), str(tmp_path)], env=env,
                       capture_output=True, text=True, timeout=240)
    say("checked child:", r.stdout.strip()[-400:], r.stderr.strip()[-400:] if r.returncode else "")
    assert r.returncode == 0, r.stderr[-2000:]
    res = json.loads(r.stdout.strip().splitlines()[-1])
    assert res["checked"]
    assert res["fwd_noplan"] == -6 and res["fwd_plan_arrays_changed"] == -6
    assert res["noalloc_noplan"] == -6 and res["noalloc_plan_arrays_changed"] == -6
    assert res["noalloc_after"] == 0
    # the normal build on the same inputs, here: bit for bit the same outputs
    ip, ix, feats = child.make_case()
    mine = child.run_all(g, ip, ix, feats)
    theirs = np.load(os.path.join(tmp_path, "checked.npz"))
    assert sorted(mine) == sorted(theirs.files)
    for k in mine:
        assert np.array_equal(mine[k].view(np.uint8), theirs[k].view(np.uint8)), k
    assert np.array_equal(np.load(os.path.join(tmp_path, "O_after.npy")).view(np.uint8), mine["O_noplan"].view(np.uint8))
