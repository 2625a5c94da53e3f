"""Build libgnn_attn.so (HIP, gfx950) in-tree with hipcc.

Run as ``python -m io_aware_sparse_amd.build`` or call :func:`build`.
Every source is compiled to its own object (in parallel), then linked.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libgnn_attn.so")
OBJ_DIR = os.path.join(ROOT, "_build", "obj")
# the checked build (GNN_CHECKED: graph validation in every call, device-side index checks)
LIB_CHECKED = os.path.join(PKG, "libgnn_attn_checked.so")
OBJ_DIR_CHECKED = os.path.join(ROOT, "_build", "obj_checked")
SOURCES = ["prep.hip", "tiles.hip", "attn.hip", "attn_tile.hip", "attn_gat.hip", "reduce.hip", "reorder.hip",
           "spmm.hip"]
HEADERS = ["device.h", "internal.h", "attn_core.h"]

COMPILE_FLAGS = [
    "-O3", "-std=c++17", "-fPIC",
    "--offload-arch=gfx950",
    # keep the compiler from forming packed fp32 instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-variable", "-Wno-unused-but-set-variable",
]
# the whole-library command line (one hipcc call over every source) is the same flags plus -shared
HIPCC_FLAGS = COMPILE_FLAGS + ["-shared"]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def sources():
    return [os.path.join(CSRC, s) for s in SOURCES]


def _jobs() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 4
    return max(1, min(len(SOURCES), n, int(os.environ.get("MAX_JOBS", "16"))))


def _filtered(stderr: str) -> str:
    # the host pass warns about the device-only target feature; keep other warnings visible
    return "\n".join(l for l in stderr.splitlines() if "packed-fp32-ops" not in l)


def build(verbose: bool = False, checked: bool = False) -> str:
    """Compile every HIP source into the package's shared library (always
    rebuilds); checked=True builds the checked variant instead."""
    obj_dir, lib = (OBJ_DIR_CHECKED, LIB_CHECKED) if checked else (OBJ_DIR, LIB)
    os.makedirs(obj_dir, exist_ok=True)
    cc = hipcc()
    inc = ["-I", os.path.join(ROOT, "include")] + (["-DGNN_CHECKED"] if checked else [])

    def compile_one(src):
        obj = os.path.join(obj_dir, os.path.basename(src) + ".o")
        cmd = [cc, *COMPILE_FLAGS, *inc, "-c", src, "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        return src, obj, cmd, r

    objs = []
    failed = False
    with ThreadPoolExecutor(max_workers=_jobs()) as ex:
        for src, obj, cmd, r in ex.map(compile_one, sources()):
            if verbose:
                print(" ".join(cmd), flush=True)
            msg = _filtered(r.stdout + r.stderr)
            if r.returncode != 0:
                sys.stderr.write(msg + "\n")
                failed = True
            elif verbose and msg.strip():
                sys.stderr.write(msg + "\n")
            objs.append(obj)
    if failed:
        raise RuntimeError("hipcc failed")
    tmp = lib + ".tmp"
    cmd = [cc, "-shared", "-fPIC", "--offload-arch=gfx950", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("hipcc link failed")
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    print(build(verbose=True))
    print(build(verbose=True, checked=True))
