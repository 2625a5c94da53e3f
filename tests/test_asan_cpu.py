"""AddressSanitizer runs on the CPU (no GPU needed).

* The fp64 oracle (oracle/oracle.c) built with -fsanitize=address and OpenMP,
  driven through every exported function (tests/asan/oracle_driver.c).
* The library's host layer: every HIP source compiled as for the product
  build, with the sanitizer on the host side only (device code is never
  instrumented), linked with a driver (tests/asan/host_layer_driver.cpp) that
  walks every entry point through its argument checks and, under the
  allocation cap, through the failure paths of plan creation and the CSR
  build. LeakSanitizer runs at exit.

Builds are cached under _build/asan/, keyed by a hash of the sources and
flags."""
import hashlib
import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "io_aware_sparse_amd", "csrc")
ASAN_DIR = os.path.join(ROOT, "_build", "asan")
INCLUDE = os.path.join(ROOT, "include")
ROCM = "/opt/rocm"
# sanitizer on the host side only; the device side is compiled as in the product build
HOST_ASAN = "-Xarch_host -fsanitize=address -Xarch_host -fno-omit-frame-pointer".split()
HIP_FLAGS = ["-O1", "-g", "-std=c++17", "-fPIC", "--offload-arch=gfx950", "-Xclang", "-target-feature", "-Xclang",
             "-packed-fp32-ops", *HOST_ASAN]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:halt_on_error=1", OMP_NUM_THREADS="3")


def _hash(files, flags):
    h = hashlib.sha256(" ".join(flags).encode())
    for f in files:
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def _run_driver(exe):
    r = subprocess.run([exe], capture_output=True, text=True, env=ENV, timeout=300)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out and "LeakSanitizer" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    return r.stdout


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not found")
def test_oracle_under_asan():
    src = [os.path.join(ROOT, "tests", "asan", "oracle_driver.c"), os.path.join(ROOT, "oracle", "oracle.c")]
    flags = ["-O1", "-g", "-std=c11", "-fopenmp", "-fsanitize=address", "-fno-omit-frame-pointer", "-fno-fast-math",
             "-ffp-contract=off"]
    d = os.path.join(ASAN_DIR, "oracle-" + _hash(src, flags))
    exe = os.path.join(d, "oracle_driver")
    if not os.path.exists(exe):
        os.makedirs(d, exist_ok=True)
        subprocess.run(["gcc", *flags, *src, "-lm", "-o", exe + ".tmp"], check=True)
        os.replace(exe + ".tmp", exe)
    assert "oracle ok" in _run_driver(exe)


@pytest.mark.skipif(not os.path.exists(os.path.join(ROCM, "bin", "hipcc")), reason="hipcc not found")
def test_host_layer_under_asan():
    sources = sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))
    headers = sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".h"))
    headers += sorted(os.path.join(INCLUDE, f) for f in os.listdir(INCLUDE))
    driver = os.path.join(ROOT, "tests", "asan", "host_layer_driver.cpp")
    d = os.path.join(ASAN_DIR, "host-" + _hash(sources + headers + [driver], HIP_FLAGS))
    exe = os.path.join(d, "host_layer_driver")
    if not os.path.exists(exe):
        os.makedirs(d, exist_ok=True)
        hipcc = os.path.join(ROCM, "bin", "hipcc")
        clang = os.path.join(ROCM, "llvm", "bin", "clang++")

        def compile_one(s):
            o = os.path.join(d, os.path.basename(s) + ".o")
            r = subprocess.run([hipcc, *HIP_FLAGS, "-I", INCLUDE, "-c", s, "-o", o], capture_output=True, text=True)
            assert r.returncode == 0, r.stderr[-3000:]
            return o

        with ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 4)) as ex:
            objs = list(ex.map(compile_one, sources))
        drv = os.path.join(d, "driver.o")
        subprocess.run([clang, "-O1", "-g", "-std=c++17", "-fsanitize=address", "-fno-omit-frame-pointer",
                        "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROCM, "include"), "-I", INCLUDE, "-c", driver,
                        "-o", drv], check=True)
        subprocess.run([clang, "-fsanitize=address", drv, *objs, "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
                        "-Wl,-rpath," + os.path.join(ROCM, "lib"), "-o", exe + ".tmp"], check=True)
        os.replace(exe + ".tmp", exe)
    assert "host layer ok" in _run_driver(exe)
