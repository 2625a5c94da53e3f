"""Build libgnn_attn.so (HIP, gfx950) in-tree with hipcc.

Run as ``python -m io_aware_sparse_amd.build`` or call :func:`build`.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libgnn_attn.so")
SOURCES = ["prep.hip", "tiles.hip", "attn.hip", "attn_tile.hip", "attn_gat.hip", "reduce.hip", "reorder.hip",
           "spmm.hip"]
HEADERS = ["device.h", "internal.h", "attn_core.h"]

HIPCC_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "-shared",
    "--offload-arch=gfx950",
    # keep the compiler from forming packed fp32 instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-variable", "-Wno-unused-but-set-variable",
]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def sources():
    return [os.path.join(CSRC, s) for s in SOURCES]


PROBE_SRC = os.path.join(CSRC, "bw_probe.hip")
PROBE = os.path.join(PKG, "bw_probe")


def build_probe(verbose: bool = False) -> str:
    """Compile the standalone bandwidth-reference executable (bench.py --bw-probe)."""
    flags = [f for f in HIPCC_FLAGS if f not in ("-fPIC", "-shared")]
    cmd = [hipcc(), *flags, PROBE_SRC, "-o", PROBE + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("hipcc failed on bw_probe.hip")
    os.replace(PROBE + ".tmp", PROBE)
    return PROBE


def build(verbose: bool = False) -> str:
    """Compile every HIP source into the package's shared library (always rebuilds)."""
    tmp = LIB + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, "-I", os.path.join(ROOT, "include"), *sources(), "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("hipcc failed")
    if verbose and r.stderr:
        # the host pass warns about the device-only target feature; keep other warnings visible
        lines = [l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l]
        if lines:
            sys.stderr.write("\n".join(lines) + "\n")
    os.replace(tmp, LIB)
    build_probe(verbose)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
