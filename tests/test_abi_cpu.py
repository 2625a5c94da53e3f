"""CPU checks of the C ABI: the library loads, exports every function the
header declares, and rejects bad arguments on the host before any HIP call
(no GPU is needed for any of these; no compute is launched)."""
import ctypes as C
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", h) for h in ("gnn_attn.h", "gnn_reduce.h", "gnn_reorder.h", "gnn_spmm.h")]


@pytest.fixture(scope="module")
def g():
    import io_aware_sparse_amd as g
    if not os.path.exists(g.LIB_PATH):
        from io_aware_sparse_amd import build
        build.build()
    g.lib()
    return g


def declared_functions():
    names = set()
    for h in HEADERS:
        src = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names |= set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", src, flags=re.M))
    return sorted(names)


def test_every_header_is_listed():
    assert sorted(os.listdir(os.path.join(ROOT, "include"))) == sorted(os.path.basename(h) for h in HEADERS)


def test_exports_every_declared_function(g):
    names = declared_functions()
    assert "gnn_attn_fwd" in names and "gatv2_attn_fwd" in names and "gnn_attn_bwd" in names
    assert "gnn_reduce_fwd" in names and "gnn_reduce_bwd" in names
    for n in names:
        assert hasattr(g.lib(), n), n
    assert sorted(g.EXPORTS) == names


def test_status_strings(g):
    for code in (0, -1, -2, -3, -4, -5, -6, -7, 99):
        assert isinstance(g.gnn_status_string(code), str)
    assert g.gnn_status_string(-3).startswith("feature pointer")
    assert "allocation-free" in g.gnn_status_string(-7)


def test_host_validation(g):
    L = g.lib()
    A = 0x10000        # aligned fake device address: never dereferenced on these paths
    # attention forward
    fwd = lambda N=10, E=20, H=2, D=32, q=A, dt=0, ip=A: L.gnn_attn_fwd(None, ip, A, N, E, H, D, q, A, A, A, None,
                                                                        0.0, dt, None)
    assert fwd(D=24) == -2 and fwd(D=0) == -2 and fwd(D=256) == -2
    assert fwd(dt=7) == -2
    assert fwd(N=-1) == -1 and fwd(E=-1) == -1 and fwd(H=0) == -1 and fwd(E=1 << 31) == -1
    assert fwd(E=(1 << 31) - (1 << 21) + 1) == -1          # edge limit: headroom for int32 positions
    assert fwd(q=A + 4) == -3
    assert fwd(ip=None) == -1
    assert L.gnn_attn_fwd(None, A, A, 10, 20, 2, 32, None, A, A, A, None, 0.0, 0, None) == -1
    assert L.gnn_attn_fwd(None, A, A, 0, 0, 2, 32, A, A, A, A, None, 0.0, 0, None) == 0   # empty graph: no-op
    # the allocation-free forward validates like gnn_attn_fwd, before any HIP call
    nfwd = lambda N=10, E=20, H=2, D=32, q=A, o=A, dt=0: L.gnn_attn_fwd_noalloc(None, A, A, N, E, H, D, q, A, A, o,
                                                                                None, 0.0, dt, None)
    assert nfwd(D=24) == -2 and nfwd(dt=7) == -2 and nfwd(N=-1) == -1 and nfwd(H=0) == -1
    assert nfwd(q=None) == -1 and nfwd(o=None) == -1 and nfwd(q=A + 4) == -3 and nfwd(o=A + 8) == -3
    assert nfwd(N=0, E=0) == 0                                                            # empty graph: no-op
    # GATv2 needs att
    assert L.gatv2_attn_fwd(None, A, A, 10, 20, 2, 32, A, A, A, None, 0.2, A, None, 0, None) == -1
    # backward needs a plan
    assert L.gnn_attn_bwd(None, A, A, 10, 20, 2, 32, A, A, A, A, A, A, A, A, A, 0.0, 0, None) == -1
    # reduction: rows of a multiple of 16 bytes, valid op / message, aligned arrays
    red = lambda N=10, E=20, F=8, x=A, arg=A, op=0, msg=0, dt=0: L.gnn_reduce_fwd(None, A, A, N, E, F, x, A, arg,
                                                                                   op, msg, dt, None)
    assert red(F=6) == -2 and red(F=4, dt=1) == -2 and red(dt=3) == -2
    assert red(F=0) == -1 and red(N=-1) == -1 and red(op=2) == -1 and red(msg=5) == -1
    assert red(x=A + 8) == -3 and red(arg=A + 4) == -3
    assert red(N=0, E=0) == 0                                                             # empty graph: no-op
    assert L.gnn_reduce_fwd(None, A, A, 10, 20, 8, None, A, None, 0, 0, 0, None) == -1
    assert L.gnn_reduce_bwd(None, A, A, 10, 20, 8, A, A, A, 0, 0, None) == -1             # needs a plan
    # reordering: sizes and method checked before the graph is touched
    assert L.gnn_reorder(A, A, 10, 20, 2, A, None) == -1 and L.gnn_reorder(A, A, -1, 0, 0, A, None) == -1
    assert L.gnn_reorder(A, A, 10, 20, 0, None, None) == -1
    assert L.gnn_reorder(A, None, 0, 0, 1, None, None) == 0                               # empty graph
    assert L.gnn_permute_graph(A, A, 10, 20, None, A, A, None) == -1
    assert L.gnn_permute_rows(A, A + 16, 10, 24, A, 0, None) == -2                        # rows of 16n bytes
    assert L.gnn_permute_rows(A, A + 8, 10, 32, A, 0, None) == -3
    assert L.gnn_permute_rows(A, A, 10, 32, A, 0, None) == -1                             # src == dst
    assert L.gnn_permute_rows(A, A + 16, 0, 32, A, 0, None) == 0
    assert L.gnn_permute_rows(None, None, 0, 32, None, 0, None) == 0                      # empty table: no-op
    # SpMM needs a plan, prepared
    assert L.gnn_spmm_prepare(None, 2, None) == -1
    assert L.gnn_spmm(None, A, A, 10, 20, 8, A, A, 0, 0, None) == -1
    assert L.gatv2_attn_bwd(None, A, A, 10, 20, 2, 32, A, A, A, A, 0.2, A, A, A, A, None, A, 0, None) == -1
    # CSR build
    e = C.c_int64()
    assert L.gnn_csr_build(A, A, 5, -1, 1, A, A, 10, C.byref(e), None) == -1
    assert L.gnn_csr_build(None, A, 5, 3, 1, A, A, 10, C.byref(e), None) == -1
    assert L.gnn_csr_build(A, A, 5, 3, 1, A, A, 10, None, None) == -1
    assert L.gnn_csr_build(A, A, 1 << 31, 3, 1, A, A, 10, C.byref(e), None) == -1
    assert L.gnn_csr_build(A, A, (1 << 31) - (1 << 21) - 2, 3, 1, A, A, 10, C.byref(e), None) == -1  # with self-loops
    # plans
    h = C.c_void_p()
    o = g.PlanOpts()
    assert L.gnn_plan_opts_default(C.byref(o)) == 0 and o.light_threshold == 512 and o.waves_per_group == 4 and o.sched_order == 2
    assert L.gnn_plan_opts_default(None) == -1
    assert L.gnn_plan_create(None, A, 10, 20, None, None, C.byref(h)) == -1
    assert L.gnn_plan_create(A, A, 10, 20, None, None, None) == -1
    assert L.gnn_plan_create(A, A, 10, (1 << 31) - (1 << 21) + 1, None, None, C.byref(h)) == -1
    assert L.gnn_reduce_fwd(None, A, A, 10, (1 << 31) - (1 << 21) + 1, 8, A, A, A, 0, 0, 0, None) == -1
    assert L.gnn_reorder(A, A, 10, (1 << 31) - (1 << 21) + 1, 0, A, None) == -1
    for field, bad in (("waves_per_group", 3), ("chunk", 0), ("light_threshold", -1), ("chunk", (1 << 18) + 1)):
        L.gnn_plan_opts_default(C.byref(o))
        setattr(o, field, bad)
        assert L.gnn_plan_create(A, A, 10, 20, C.byref(o), None, C.byref(h)) == -1, field
    assert L.gnn_plan_export(None, None) == -1
    assert L.gnn_plan_destroy(None) == -1
    assert L.gnn_plan_set_timing(None, 1) == -1
    n = C.c_int32()
    assert L.gnn_plan_timing_read(None, 0, None, None, None, C.byref(n)) == -1


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    import io_aware_sparse_amd as g
    monkeypatch.setattr(g, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(g, "_lib", None)
    with pytest.raises(RuntimeError, match="HIP library missing"):
        g.lib()


def test_alloc_cap_forces_oom_before_any_hip_call(g, monkeypatch):
    """GNN_ALLOC_CAP_BYTES (a test hook) refuses every device allocation larger
    than the cap before hipMalloc is called: plan creation and the CSR build
    then fail cleanly with GNN_ERR_OOM, naming the cap, with no GPU needed."""
    L = g.lib()
    A = 0x10000
    h = C.c_void_p()
    e = C.c_int64()
    monkeypatch.setenv("GNN_ALLOC_CAP_BYTES", "0")
    assert L.gnn_plan_create(A, A, 10, 20, None, None, C.byref(h)) == -4
    assert h.value is None                                     # *plan_out untouched on failure
    assert "GNN_ALLOC_CAP_BYTES=0" in g.gnn_status_string(-4)
    assert L.gnn_csr_build(A, A, 5, 3, 1, A, A, 10, C.byref(e), None) == -4
    monkeypatch.setenv("GNN_ALLOC_CAP_BYTES", "32")            # below the first 64-byte request
    assert L.gnn_plan_create(A, A, 10, 20, None, None, C.byref(h)) == -4
    assert "GNN_ALLOC_CAP_BYTES=32" in g.gnn_status_string(-4)
    with pytest.raises(g.GnnError) as err:
        g._check(L.gnn_plan_create(A, A, 10, 20, None, None, C.byref(h)), "gnn_plan_create")
    assert err.value.status == -4 and "GNN_ERR_OOM" in str(err.value)


def test_binding_structs_match_the_header(tmp_path):
    """The binding's ctypes mirrors of gnn_plan_opts and gnn_plan_info have
    the header's size and every field's offset (a C program built from the
    header with the host compiler prints them)."""
    import shutil
    import subprocess
    import io_aware_sparse_amd as g
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no host C compiler")
    lines = []
    for cname, py in (("gnn_plan_opts", g.PlanOpts), ("gnn_plan_info", g.PlanInfo)):
        lines.append(f'printf("{cname} size %zu\\n", sizeof({cname}));')
        for f, _ in py._fields_:
            lines.append(f'printf("{cname} {f} %zu\\n", offsetof({cname}, {f}));')
    src = tmp_path / "layout.c"
    src.write_text("#include <stdio.h>\n#include <stddef.h>\n#include \"gnn_attn.h\"\nint main(void) {\n"
                   + "\n".join(lines) + "\nreturn 0;\n}\n")
    exe = tmp_path / "layout"
    r = subprocess.run([cc, "-I", os.path.join(ROOT, "include"), "-I", "/opt/rocm/include", "-D__HIP_PLATFORM_AMD__",
                        str(src), "-o", str(exe)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    got = {}
    for line in subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout.splitlines():
        s, f, v = line.split()
        got[(s, f)] = int(v)
    for cname, py in (("gnn_plan_opts", g.PlanOpts), ("gnn_plan_info", g.PlanInfo)):
        assert got[(cname, "size")] == C.sizeof(py), cname
        for f, _ in py._fields_:
            assert got[(cname, f)] == getattr(py, f).offset, (cname, f)
