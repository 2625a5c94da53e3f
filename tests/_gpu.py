"""Helpers for GPU parity tests: move seeded inputs to the device, call the
library through its C ABI, and compare with the oracle.

Tolerances: max condition-scaled error 1e-4 (fp32 inputs) or 2e-2 (bf16),
the scale being the oracle's sum of absolute terms of each output."""
import sys

import numpy as np

TOL = {"f32": 1e-4, "bf16": 2e-2}


def say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def check(name, x, ref, scale, dtype, extra=""):
    """Assert the condition-scaled error of x against the oracle's ref is
    within the tolerance of dtype; print it with the plain normwise error
    max|x - r| / max|r| beside it. Returns the scaled error."""
    import oracle
    err = oracle.scaled_error(x, ref, scale)
    nw = oracle.normwise_error(x, ref)
    say(f"  {name}: scaled err {err:.3e}, normwise {nw:.3e}{extra} (tol {TOL[dtype]:.0e})")
    assert err <= TOL[dtype], (name, err)
    return err


def torch():
    import torch as t
    return t


def dev_feat(values_f32: np.ndarray, dtype: str):
    """Device tensor holding `values_f32` (already representable in dtype)."""
    t = torch()
    x = t.from_numpy(np.ascontiguousarray(values_f32, np.float32)).cuda()
    return x if dtype == "f32" else x.to(t.bfloat16)


def dev_i32(a):
    t = torch()
    return t.from_numpy(np.ascontiguousarray(a, np.int32)).cuda()


def host(x) -> np.ndarray:
    t = torch()
    return x.detach().to(t.float32).cpu().numpy().astype(np.float64) if x.dtype != t.float32 \
        else x.detach().cpu().numpy().astype(np.float64)


def round_like(x: np.ndarray, dtype: str) -> np.ndarray:
    """Values of x after storage in dtype (bf16: round-to-nearest-even)."""
    if dtype == "f32":
        return x.astype(np.float32)
    t = torch()
    return t.from_numpy(np.ascontiguousarray(x, np.float32)).to(t.bfloat16).to(t.float32).numpy()


def rand_feats(rng, n, h, d, dtype, k=3, scale=1.0):
    return [round_like(rng.standard_normal((n, h, d)) * scale, dtype) for _ in range(k)]
